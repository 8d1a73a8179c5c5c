// fp32 blockwise exact attention (ring prefill and single ring step) for gfx950.
//
// Same protocol as the bf16 kernel: every KV tile updates the per-row running
// maximum and exp-sum, rescales the output accumulator and adds the tile's
// contribution (page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条
// 超长序列", §"最容易被忽略的细节"; blocks in the ring order of §"KV 在 Ring 中如何
// 流动"). Everything stays in fp32, nothing is rounded to a narrower type: this path
// exists for fp32 inputs, whose tolerance no bf16 product could meet.
//
// Both products are dense contractions, so they run on the fp32 matrix cores:
// v_mfma_f32_32x32x2_f32 (or 16x16x4) multiplies fp32 blocks into an fp32
// accumulator at 64 FLOP per clock per SIMD, twice what the vector ALUs reach with
// unpacked FMAs, and leaves the ALUs to the softmax.
//
// Workgroup: 8 waves = NR blocks of M query rows x NS key streams (M = 32 or 16,
// the product shape). A key tile of M NS keys goes from HBM straight into LDS
// (buffer_load ... lds, double-buffered, one barrier per tile); the wave of (row
// block r, stream s) takes the tile's s-th M keys for its M rows. With G = 64 / M
// lane groups, lane L holds query row L % M, and per wave and sub-block:
//   Sᵀ = K Qᵀ    D_qk / G products. The stationary B operand holds dimensions
//                 (L / M) D_qk / G + step of the lane's row; the A operand is the
//                 same dimension of key L % M, read from padded LDS rows four steps
//                 at a time. Lane L ends with the row's scores against the M² / 64
//                 keys (v / 4) 4 G + 4 (L / M) + v % 4 (the accumulator layout).
//   softmax      row max and sum over the lane's scores and the G lanes of the row
//                 (v_permlane32_swap, and a 16-lane xor shuffle when G = 4);
//                 running max, rescale of Oᵀ by 2^(m - m'), P = 2^(s scale log2 e -
//                 m') in place.
//   Oᵀ += Vᵀ Pᵀ  per M output columns, M² / 64 products: product t pairs the lane's
//                 score t (key (t / 4) 4 G + 4 (L / M) + t % 4) with that key's V
//                 value of column L % M, read from LDS.
// The NS streams' states of a row block meet in LDS at the end: with M' the largest
// running max, l = sum l_s 2^(m_s - M') and O = sum O_s 2^(m_s - M'), the merge of
// partial softmax states over disjoint key sets.
#include <type_traits>

#include "common.hpp"

namespace ra {

enum { F32_RING = 0, F32_STEP = 1 };

// One fp32 MFMA shape: M x M outputs from an M x K by a K x M product, K = 256 / M
// (v_mfma_f32_32x32x2_f32 or v_mfma_f32_16x16x4_f32, both 64 FLOP per clock per
// SIMD). The A and B operands take row (column) L % M and k index L / M of lane L;
// the accumulator gives lane L column L % M and rows (v / 4) 4 G + 4 (L / M) + v % 4,
// v < M² / 64, with G = 64 / M lane groups.
template <int M>
struct F32Mfma;
template <>
struct F32Mfma<32> {
  typedef f32x16 acc;
  static __device__ __forceinline__ acc mma(float a, float b, acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};
template <>
struct F32Mfma<16> {
  typedef f32x4 acc;
  static __device__ __forceinline__ acc mma(float a, float b, acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// max / sum of v over the G lanes 16 apart that hold one row (G = 2: the two
// halves; G = 4: lanes L, L ^ 16, L ^ 32, L ^ 48). Every lane of the row gets the
// same value: each step combines two values with a commutative operation.
template <int G>
__device__ __forceinline__ float groups_max(float v) {
  if constexpr (G == 4) v = fmaxf(v, shfl_xor_f(v, 16));
  return row_max_halves(v);
}
template <int G>
__device__ __forceinline__ float groups_sum(float v) {
  if constexpr (G == 4) v += shfl_xor_f(v, 16);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DQK, int DV, int M_>
struct F32Cfg {
  static constexpr int M = M_, G = 64 / M;
  // key streams: a tile holds NS sub-blocks of M keys, and two buffers of it fit
  // 160 KB of LDS
  static constexpr int NS = (DQK + DV <= 128 ? 4 : 2) * (32 / M);
  static constexpr int NR = 8 / NS;                 // M-row blocks per workgroup
  static constexpr int THREADS = 512;
  static constexpr int BQ = M * NR, BK = M * NS;    // query rows, keys per tile
  // padded LDS rows (floats): 16 consecutive K rows start 4 banks apart, so the
  // 16-byte reads of a quarter wave (16 rows, same columns) are conflict-free. The
  // 32-bit V reads of a wave take M consecutive columns in each of G rows 4 apart
  // (rows 4 g + const): rows 4 apart start 32 banks apart when M = 32 and 16 banks
  // apart when M = 16, so the wave's 64 reads hit 64 distinct banks
  static constexpr int KS = DQK + 4, VS = DV + (M == 32 ? 8 : 4);
  static constexpr int K_TILE = padded_tile_bytes(BK, KS * 4) / 4;   // floats per buffer
  static constexpr int V_TILE = padded_tile_bytes(BK, VS * 4) / 4;
  static constexpr int DS = DQK / G;      // score products per sub-block
  static constexpr int SV = M * M / 64;   // scores per lane per sub-block (= PV products per output tile)
  static constexpr int MT = DV / M;       // output tiles of M columns
  static constexpr int MERGE = M * DV + 128;   // one wave's O, m, l in the stream merge
  static_assert(NS * NR == 8, "eight waves");
  static_assert(2 * (K_TILE + V_TILE) * 4 <= 160 * 1024, "LDS");
  static_assert((NS - 1) * NR * MERGE <= 2 * (K_TILE + V_TILE), "merge area");
};

// A workgroup's query tile (rows, positions, head) and its key-tile schedule.
template <int BQ, int BK, int MODE>
struct F32Work {
  int bh, b, g, row_base, row_end, ntiles;
  long long pos_base;
  RingTiles ring;
  size_t kvh;
  long long k_pos0;
  int Sk;
  // false: the tile sees no key (step mode), nothing to do
  __device__ __forceinline__ bool init(const PrefillArgs& a) {
    const int tiles_per_head = (MODE == F32_RING ? a.nq : 1) * a.n_qtiles;
    // the heaviest causal tiles of every head first: workgroup x takes head x % (B
    // Hq) and the (x / (B Hq))-th heaviest of its tiles. (Head by head, heaviest
    // first inside each head, ran 1.8x slower at 8 heads and 512 workgroups.)
    const int nbh = a.B * a.Hq;
    bh = blockIdx.x % nbh;
    const int gt = tiles_per_head - 1 - (int)(blockIdx.x / nbh);
    b = bh / a.Hq;
    const int hq = bh - b * a.Hq;
    g = hq / a.group;
    int part = 0, qt = gt;
    if (MODE == F32_RING) {
      part = gt / a.n_qtiles;
      qt = gt - part * a.n_qtiles;
    }
    if (MODE == F32_RING) {
      row_base = part * a.Sp + qt * BQ;
      row_end = part * a.Sp + a.Sp;
      // striped causal: virtual query position = local row (see RingTiles)
      pos_base = (a.causal && a.striped ? 0LL : (long long)(a.q_part0 + part) * a.Sp) + qt * BQ;
    } else {
      row_base = qt * BQ;
      row_end = a.q_rows;
      pos_base = a.q_pos0 + row_base;
    }
    const int last_row = min(row_base + BQ, row_end) - 1;
    const long long last_pos = pos_base + (last_row - row_base);
    kvh = (size_t)(b * a.Hkv + g) * a.kv_rows;
    k_pos0 = a.k_pos0;
    Sk = a.Sk;
    if (MODE == F32_RING) {
      ring.init(a.q_part0 + part, a.P, a.Sp, BK, a.causal != 0, a.striped != 0, last_row - part * a.Sp);
      ntiles = ring.ntiles;
    } else {
      long long kmax = a.Sk;
      if (a.causal) kmax = min(kmax, last_pos - a.k_pos0 + 1);
      if (kmax <= 0) return false;
      ntiles = (int)((kmax + BK - 1) / BK);
    }
    return true;
  }
  // tile n -> first key row, position of that key, valid keys (random access)
  __device__ __forceinline__ void tile_at(int n, int& krow0, long long& kpos0, int& nvalid) const {
    if (MODE == F32_RING) {
      ring.tile(n, krow0, kpos0, nvalid);
    } else {
      krow0 = n * BK;
      kpos0 = k_pos0 + (long long)n * BK;
      nvalid = min(BK, Sk - n * BK);
    }
  }
};

template <int DQK, int DV, int MODE, int M>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_f32_kernel(PrefillArgs a) {
  using C = F32Cfg<DQK, DV, M>;
  using MM = F32Mfma<M>;
  using acc_t = typename MM::acc;
  constexpr int NR = C::NR, NS = C::NS, BQ = C::BQ, BK = C::BK, KS = C::KS, VS = C::VS;
  constexpr int G = C::G, DS = C::DS, SV = C::SV, MT = C::MT;
  __shared__ __attribute__((aligned(1024))) float smem[2 * (C::K_TILE + C::V_TILE)];

  const int lane = threadIdx.x & 63, lm = lane % M, g = lane / M;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int rb = wave % NR, stream = wave / NR;
  // accumulator row (key, or output column) of element v for this lane's group
  auto acc_row = [&](int v) __attribute__((always_inline)) { return (v >> 2) * 4 * G + 4 * g + (v & 3); };

  F32Work<BQ, BK, MODE> w;
  if (!w.init(a)) return;
  const int ntiles = w.ntiles;

  // this wave's rows: M from row_base + M rb (fewer, or none, at a ragged end)
  const int wrow0 = w.row_base + M * rb;
  const int wrows = min(M, w.row_end - wrow0);
  const long long wpos0 = w.pos_base + M * rb;
  const int row = wrow0 + lm;
  const bool row_ok = lm < wrows;
  const long long qpos = wpos0 + lm;

  // stationary Q: dimensions g DS .. g DS + DS - 1 of the lane's row
  float q[DS];
  {
    const float* qr = (const float*)a.q + ((size_t)w.bh * a.q_rows + row) * DQK + g * DS;
#pragma unroll
    for (int c = 0; c < DS / 4; ++c) {
      const float4 x = row_ok ? *(const float4*)(qr + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[4 * c] = x.x;
      q[4 * c + 1] = x.y;
      q[4 * c + 2] = x.z;
      q[4 * c + 3] = x.w;
    }
  }

  // running state of row lm: max (log2 units), exp-sum, Oᵀ accumulators (lane holds
  // columns M mt + acc_row(v))
  float m = kNegInf, l = 0.f;
  acc_t o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = acc_t{};
  if (MODE == F32_STEP && stream == 0 && row_ok) {
    // the running state (O normalised, LSE) enters through stream 0 as m = LSE, l = 1
    const size_t r = (size_t)w.bh * a.q_rows + row;
    const float lin = a.lse_acc[r];
    if (lin != kNegInf) {
      m = lin * kLog2e;
      l = 1.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v4 = 0; v4 < SV; v4 += 4) {
          const float4 x = *(const float4*)(a.o_acc + r * DV + M * mt + acc_row(v4));
          o[mt][v4] = x.x;
          o[mt][v4 + 1] = x.y;
          o[mt][v4 + 2] = x.z;
          o[mt][v4 + 3] = x.w;
        }
    }
  }

  // direct HBM -> LDS tile loads
  const u32x4 kdesc = raw_desc((const float*)a.k + w.kvh * DQK, (unsigned)((size_t)a.kv_rows * DQK * 4));
  const u32x4 vdesc = raw_desc((const float*)a.v + w.kvh * DV, (unsigned)((size_t)a.kv_rows * DV * 4));
  const unsigned k_last = (unsigned)((size_t)a.kv_rows * DQK * 4 - 16);
  const unsigned v_last = (unsigned)((size_t)a.kv_rows * DV * 4 - 16);
  const unsigned k_lds = lds_addr(smem), v_lds = lds_addr(smem + 2 * C::K_TILE);
  PaddedTileDma<BK, DQK * 4, KS * 4, 8> kpad;
  PaddedTileDma<BK, DV * 4, VS * 4, 8> vpad;
  kpad.init(wave, lane);
  vpad.init(wave, lane);
  auto dma = [&](int n, int buf) __attribute__((always_inline)) {
    int krow0, nvalid;
    long long kpos0;
    w.tile_at(n, krow0, kpos0, nvalid);
    kpad.issue(wave, k_lds + (unsigned)(buf * C::K_TILE * 4), (unsigned)krow0 * (DQK * 4), k_last, kdesc);
    vpad.issue(wave, v_lds + (unsigned)(buf * C::V_TILE * 4), (unsigned)krow0 * (DV * 4), v_last, vdesc);
  };

  // one sub-block: keys kb .. kb + M - 1 of the tile in buffer buf, positions from
  // kpos; nv of them valid
  auto compute = [&](int buf, int kb, long long kpos, int nv, bool need_mask) __attribute__((always_inline)) {
    const float* kt = smem + buf * C::K_TILE + (kb + lm) * KS + g * DS;
    acc_t s = acc_t{};
#pragma unroll
    for (int c = 0; c < DS / 4; ++c) {
      const float4 kv = *(const float4*)(kt + 4 * c);
      s = MM::mma(kv.x, q[4 * c], s);
      s = MM::mma(kv.y, q[4 * c + 1], s);
      s = MM::mma(kv.z, q[4 * c + 2], s);
      s = MM::mma(kv.w, q[4 * c + 3], s);
    }
    if (need_mask) {
#pragma unroll
      for (int v = 0; v < SV; ++v) {
        const int key = acc_row(v);
        const bool ok = key < nv && (!a.causal || kpos + key <= qpos);
        s[v] = ok ? s[v] : kNegInf;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int v = 1; v < SV; ++v) mx = fmaxf(mx, s[v]);
    mx = groups_max<G>(mx);
    const float mnew = fmaxf(m, mx * a.scale_log2);
    const float muse = mnew == kNegInf ? 0.f : mnew;
    const float alpha = exp2_hw(m - muse);
    m = mnew;
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < SV; ++v) {
      s[v] = exp2_hw(fmaf(s[v], a.scale_log2, -muse));
      rs += s[v];
    }
    l = fmaf(l, alpha, groups_sum<G>(rs));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
    // product t takes key acc_row(t) of this lane's group: its own P value t and
    // that key's V value of column lm
    const float* vt = smem + 2 * C::K_TILE + buf * C::V_TILE + (kb + 4 * g) * VS + lm;
#pragma unroll
    for (int t = 0; t < SV; ++t) {
      const int kr = (t >> 2) * 4 * G + (t & 3);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = MM::mma(vt[kr * VS + M * mt], s[t], o[mt]);
    }
  };

  if (ntiles > 0) dma(0, 0);
  wait_vmem();
  __syncthreads();
  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    // buffer buf ^ 1 held tile n - 1, which every wave finished before the barrier
    if (n + 1 < ntiles) dma(n + 1, buf ^ 1);
    int krow0, nvalid;
    long long kpos0;
    w.tile_at(n, krow0, kpos0, nvalid);
    const int kb = M * stream;
    const long long kpos = kpos0 + kb;
    // wave-uniform: no valid key or row (skip), or some key masked for some row
    bool skip = kb >= nvalid || wrows <= 0;
    if (a.causal) skip = skip || kpos > wpos0 + wrows - 1;
    const bool need_mask = kb + M > nvalid || (a.causal && kpos + M - 1 > wpos0);
    if (!skip) compute(buf, kb, kpos, nvalid - kb, need_mask);
    wait_vmem();   // this wave's loads of tile n + 1 have landed
    __syncthreads();
  }

  // merge of the streams (the tile buffers are free after the last barrier)
  if constexpr (NS > 1) {
    if (stream > 0) {
      float* mb = smem + ((stream - 1) * NR + rb) * C::MERGE;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < SV; ++v) mb[(SV * mt + v) * 64 + lane] = o[mt][v];
      if (g == 0) {
        mb[M * DV + lm] = m;
        mb[M * DV + 64 + lm] = l;
      }
    }
    __syncthreads();
    if (stream > 0) return;
    float Mx = m;
#pragma unroll
    for (int s = 1; s < NS; ++s) Mx = fmaxf(Mx, smem[((s - 1) * NR + rb) * C::MERGE + M * DV + lm]);
    const float w0 = m == kNegInf ? 0.f : exp2_hw(m - Mx);
    l *= w0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] *= w0;
#pragma unroll
    for (int s = 1; s < NS; ++s) {
      const float* mb = smem + ((s - 1) * NR + rb) * C::MERGE;
      const float ms = mb[M * DV + lm];
      const float ws = ms == kNegInf ? 0.f : exp2_hw(ms - Mx);
      l = fmaf(mb[M * DV + 64 + lm], ws, l);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < SV; ++v) o[mt][v] = fmaf(mb[(SV * mt + v) * 64 + lane], ws, o[mt][v]);
    }
    m = Mx;
  }

  if (!row_ok) return;
  const size_t r = (size_t)w.bh * a.q_rows + row;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? (m + log2_hw(l)) * kLn2 : kNegInf;
  float* out = MODE == F32_RING ? (float*)a.o : a.o_acc;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v4 = 0; v4 < SV; v4 += 4)
      *(float4*)(out + r * DV + M * mt + acc_row(v4)) =
          make_float4(o[mt][v4] * inv, o[mt][v4 + 1] * inv, o[mt][v4 + 2] * inv, o[mt][v4 + 3] * inv);
  if (g == 0) {
    if (MODE == F32_RING)
      a.lse[r] = lse;
    else
      a.lse_acc[r] = lse;
  }
}

template <int DQK, int DV, int MODE, int M>
static hipError_t launch_f32_as(PrefillArgs a, hipStream_t st) {
  using C = F32Cfg<DQK, DV, M>;
  const int rows_per_part = MODE == F32_RING ? a.Sp : a.q_rows;
  a.n_qtiles = (rows_per_part + C::BQ - 1) / C::BQ;
  const long long tiles = (long long)a.B * a.Hq * (MODE == F32_RING ? a.nq : 1) * a.n_qtiles;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_kernel<DQK, DV, MODE, M>), dim3((unsigned)tiles), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

// 32 x 32 products (128 query rows per workgroup; 64 at D_qk = D_v = 64) when the
// launch has at least two such workgroups per CU; otherwise 16 x 16 products (32 or
// 16 rows per workgroup, the keys of a tile split over 4 or 8 streams), which put
// four times the workgroups on a small launch. Measured: 32 x 32 runs large launches
// 1.2-1.4x faster; 16 x 16 runs 16 to 40 workgroups' worth 2-2.6x faster.
template <int DQK, int DV, int MODE>
static hipError_t launch_f32(PrefillArgs a, hipStream_t st) {
  using C = F32Cfg<DQK, DV, 32>;
  const int rows_per_part = MODE == F32_RING ? a.Sp : a.q_rows;
  const long long wgs32 = (long long)a.B * a.Hq * (MODE == F32_RING ? a.nq : 1) * ((rows_per_part + C::BQ - 1) / C::BQ);
  if (wgs32 >= 512) return launch_f32_as<DQK, DV, MODE, 32>(a, st);
  return launch_f32_as<DQK, DV, MODE, 16>(a, st);
}

hipError_t prefill_f32(const PrefillArgs& a, int dqk, int dv, int step_mode, hipStream_t st) {
#define RA_F32_CASE(X, Y)                                                                      \
  if (dqk == X && dv == Y)                                                                     \
    return step_mode ? launch_f32<X, Y, F32_STEP>(a, st) : launch_f32<X, Y, F32_RING>(a, st);
  RA_F32_CASE(64, 64)
  RA_F32_CASE(64, 128)
  RA_F32_CASE(128, 64)
  RA_F32_CASE(128, 128)
#undef RA_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace ra
