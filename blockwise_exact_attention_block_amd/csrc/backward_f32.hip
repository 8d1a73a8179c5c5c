// Backward pass of blockwise exact attention for fp32 inputs on gfx950, on the fp32
// matrix cores.
//
// The same gradients as the bf16 backward (the exact gradients of O = softmax(scale *
// Q K^T) V over the visible keys, page "长上下文的第一性挑战", §挑战 1, eq.
// lc-ch-attention; computed one (query block, KV block) pair at a time from the
// queries' saved row LSE and delta = rowsum(dO o O), so a ring backward sums such
// pairs; page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条超长序列",
// §什么时候值得引入 Context Parallelism). With P = exp(scale q k - LSE):
//     dV += P^T dO,  dS = P o (dO V^T - delta),  dQ += scale dS K,  dK += scale dS^T Q.
// Everything stays in fp32: no product rounds P or dS, so this path meets the fp32
// tolerance that the bf16 kernels cannot.
//
// Every product runs on v_mfma_f32_16x16x4_f32 (a 16 x 4 by 4 x 16 fp32 block into a
// 16 x 16 fp32 accumulator, 64 FLOP per clock per SIMD). Lane L of a wave works for
// row (or key) L % 16 of its 16 x 16 block and lane group g = L / 16: an operand
// "stationary" in a lane holds dimensions g D / 4 .. g D / 4 + D / 4 - 1 of that row,
// and an accumulator gives the lane column L % 16 and rows 4 g .. 4 g + 3.
//
// Three kernels:
//   * bwd_delta_f32_kernel: delta per query row, 16 lanes per row.
//   * bwd_dq_f32_kernel (8 waves): 64 query rows of one (batch, head) = 4 row blocks
//     x 2 key streams (32 rows = 2 x 4 in launches of fewer 64-row workgroups than
//     CUs); K / V tiles of 16 keys per stream go from HBM into LDS (direct loads,
//     double-buffered). A wave keeps its 16 rows' Q and dO stationary, forms
//     Sᵀ = K Qᵀ and dPᵀ = V dOᵀ for 16 keys (lane: row L % 16, keys 4 g + v), P and
//     dS in registers, then dQᵀ += Kᵀ dSᵀ with the lane's dS values as the B operand
//     and K read back from LDS as A. The streams' sums meet in LDS at the end.
//   * bwd_dkdv_f32_kernel (8 waves): 32 keys of one (batch, KV head) = 2 key blocks
//     x 4 query streams. A wave keeps its 16 keys' K and V stationary; it walks the
//     group's query heads and the query tiles of 64 rows that can see them (Q, dO,
//     LSE and delta in LDS, double-buffered), forms S = Q Kᵀ and dP = dO Vᵀ (lane:
//     key L % 16, rows 4 g + v), P and dS, then dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS with
//     dO and Q read back from LDS. Under a causal mask a workgroup takes key tiles
//     kt and n - 1 - kt, which balances the work. The query streams' sums meet in
//     LDS at the end.
// LDS rows are padded by 4 floats, so the 16-byte operand reads of 16 rows at one
// column and the 4-byte reads of rows 4 apart at 16 consecutive columns are both
// free of bank conflicts. Every sum runs in a fixed order, so results repeat bit for
// bit.
#include "common.hpp"

namespace ra {

// ---- delta = rowsum(dO o O) -----------------------------------------------------------
__global__ void __launch_bounds__(256)
bwd_delta_f32_kernel(const float* o, const float* dout, float* delta, long long rows, int Dv) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int L = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    for (int c = L; c < Dv / 4; c += 16) {
      const float4 x = *(const float4*)(o + row * Dv + 4 * c);
      const float4 y = *(const float4*)(dout + row * Dv + 4 * c);
      acc = fmaf(x.x, y.x, acc);
      acc = fmaf(x.y, y.y, acc);
      acc = fmaf(x.z, y.z, acc);
      acc = fmaf(x.w, y.w, acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += shfl_xor_f(acc, m);
  if (row < rows && L == 0) delta[row] = acc;
}

__device__ __forceinline__ f32x4 mma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D / 4 consecutive floats from global memory (zero when !ok) into registers
template <int N>
__device__ __forceinline__ void load_vec(float (&x)[N], const float* p, bool ok) {
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    const float4 v = ok ? *(const float4*)(p + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    x[4 * c] = v.x;
    x[4 * c + 1] = v.y;
    x[4 * c + 2] = v.z;
    x[4 * c + 3] = v.w;
  }
}

// acc += A B over N steps: A from LDS (16-byte reads, four steps each), B stationary
template <int N>
__device__ __forceinline__ f32x4 chain(const float* lds, const float (&b)[N], f32x4 acc) {
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    const float4 x = *(const float4*)(lds + 4 * c);
    acc = mma16_f32(x.x, b[4 * c], acc);
    acc = mma16_f32(x.y, b[4 * c + 1], acc);
    acc = mma16_f32(x.z, b[4 * c + 2], acc);
    acc = mma16_f32(x.w, b[4 * c + 3], acc);
  }
  return acc;
}

// ---- dQ -------------------------------------------------------------------------------
template <int DQK, int DV, int NR_>
struct F32DqCfg {
  static constexpr int NR = NR_, NS = 8 / NR_;        // 16-row blocks x key streams
  static constexpr int BQ = 16 * NR, BK = 16 * NS;    // query rows per workgroup, keys per tile
  static constexpr int KS = DQK + 4, VS = DV + 4;
  static constexpr int K_TILE = padded_tile_bytes(BK, KS * 4) / 4;   // floats per buffer
  static constexpr int V_TILE = padded_tile_bytes(BK, VS * 4) / 4;
  static constexpr int DT = DQK / 16;                 // dQ output tiles of 16 columns
  static constexpr int MERGE = 16 * DQK;              // one wave's dQ partial sums
  static_assert(NR * NS == 8, "eight waves");
  static_assert((NS - 1) * NR * MERGE <= 2 * (K_TILE + V_TILE), "merge area");
};

template <int DQK, int DV, int NR_>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_f32_kernel(BwdArgs a) {
  using C = F32DqCfg<DQK, DV, NR_>;
  constexpr int NR = C::NR, NS = C::NS, BQ = C::BQ, BK = C::BK, KS = C::KS, VS = C::VS, DT = C::DT;
  __shared__ __attribute__((aligned(1024))) float smem[2 * (C::K_TILE + C::V_TILE)];
  const int lane = threadIdx.x & 63, lm = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int rb = wave % NR, stream = wave / NR;

  // workgroup x: head x % (B Hq) and the (x / (B Hq))-th heaviest of its query tiles
  const int nbh = a.B * a.Hq;
  const int bh = blockIdx.x % nbh;
  const int qt = a.n_tiles - 1 - (int)(blockIdx.x / nbh);
  const int b = bh / a.Hq, hq = bh - b * a.Hq, kvg = hq / a.group;
  const int row_base = qt * BQ;
  const int last_row = min(row_base + BQ, a.Sq) - 1;
  long long kmax = a.Sk;
  if (a.causal) kmax = min(kmax, a.q_pos0 + last_row - a.k_pos0 + 1);
  if (kmax <= 0) return;   // no key of the block is visible to this tile
  const int ntiles = (int)((kmax + BK - 1) / BK);

  const int wrow0 = row_base + 16 * rb;
  const int wrows = min(16, a.Sq - wrow0);
  const long long wpos0 = a.q_pos0 + wrow0;
  const int row = wrow0 + lm;
  const bool row_ok = lm < wrows;
  const long long qpos = wpos0 + lm;

  float q[DQK / 4], dout[DV / 4];
  load_vec(q, (const float*)a.q + ((size_t)bh * a.Sq + row) * DQK + g * (DQK / 4), row_ok);
  load_vec(dout, (const float*)a.dout + ((size_t)bh * a.Sq + row) * DV + g * (DV / 4), row_ok);
  // a row past the block, or with no visible key, gets P = 0 (exp2(s - inf))
  float lse2 = __builtin_huge_valf(), dl = 0.f;
  if (row_ok) {
    const float l = a.lse[(size_t)bh * a.Sq + row];
    if (l != kNegInf) lse2 = l * kLog2e;
    dl = a.delta[(size_t)bh * a.Sq + row];
  }
  f32x4 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = f32x4{};

  const size_t kvh = (size_t)(b * a.Hkv + kvg) * a.Sk;
  const u32x4 kdesc = raw_desc((const float*)a.k + kvh * DQK, (unsigned)((size_t)a.Sk * DQK * 4));
  const u32x4 vdesc = raw_desc((const float*)a.v + kvh * DV, (unsigned)((size_t)a.Sk * DV * 4));
  const unsigned k_last = (unsigned)((size_t)a.Sk * DQK * 4 - 16), v_last = (unsigned)((size_t)a.Sk * DV * 4 - 16);
  const unsigned k_lds = lds_addr(smem), v_lds = lds_addr(smem + 2 * C::K_TILE);
  PaddedTileDma<BK, DQK * 4, KS * 4, 8> kpad;
  PaddedTileDma<BK, DV * 4, VS * 4, 8> vpad;
  kpad.init(wave, lane);
  vpad.init(wave, lane);
  auto dma = [&](int n, int buf) __attribute__((always_inline)) {
    kpad.issue(wave, k_lds + (unsigned)(buf * C::K_TILE * 4), (unsigned)(n * BK) * (DQK * 4), k_last, kdesc);
    vpad.issue(wave, v_lds + (unsigned)(buf * C::V_TILE * 4), (unsigned)(n * BK) * (DV * 4), v_last, vdesc);
  };

  dma(0, 0);
  wait_vmem();
  __syncthreads();
  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    if (n + 1 < ntiles) dma(n + 1, buf ^ 1);
    const int kb = 16 * stream;
    const int nv = min(BK, a.Sk - n * BK) - kb;   // valid keys of this sub-block
    const long long kpos = a.k_pos0 + (long long)n * BK + kb;
    bool skip = nv <= 0 || wrows <= 0;
    if (a.causal) skip = skip || kpos > wpos0 + wrows - 1;
    const bool need_mask = nv < 16 || (a.causal && kpos + 15 > wpos0);
    if (!skip) {
      const float* kt = smem + buf * C::K_TILE;
      const float* vt = smem + 2 * C::K_TILE + buf * C::V_TILE;
      // Sᵀ and dPᵀ: lane holds row lm against keys 4 g + v
      const f32x4 s = chain(kt + (kb + lm) * KS + g * (DQK / 4), q, f32x4{});
      const f32x4 dp = chain(vt + (kb + lm) * VS + g * (DV / 4), dout, f32x4{});
      float ds[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = 4 * g + v;
        const bool vis = !need_mask || (key < nv && (!a.causal || kpos + key <= qpos));
        const float p = vis ? exp2_hw(fmaf(s[v], a.scale_log2, -lse2)) : 0.f;
        ds[v] = p * (dp[v] - dl);
      }
      // dQᵀ += Kᵀ dSᵀ: product t takes key 4 g + t, K read at column 16 dt + lm
      const float* kc = kt + (kb + 4 * g) * KS + lm;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int d = 0; d < DT; ++d) dq[d] = mma16_f32(kc[t * KS + 16 * d], ds[t], dq[d]);
    }
    wait_vmem();   // this wave's loads of tile n + 1 have landed
    __syncthreads();
  }

  // the key streams' sums meet in LDS (the tile buffers are free after the last barrier)
  if constexpr (NS > 1) {
    if (stream > 0) {
      float* mb = smem + ((stream - 1) * NR + rb) * C::MERGE;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int v = 0; v < 4; ++v) mb[(4 * d + v) * 64 + lane] = dq[d][v];
    }
    __syncthreads();
    if (stream > 0) return;
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2) {
      const float* mb = smem + ((s2 - 1) * NR + rb) * C::MERGE;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int v = 0; v < 4; ++v) dq[d][v] += mb[(4 * d + v) * 64 + lane];
    }
  }
  if (!row_ok) return;
  float* dqp = a.dq + ((size_t)bh * a.Sq + row) * DQK + 4 * g;
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    float4 cur = *(const float4*)(dqp + 16 * d);
    cur.x = fmaf(a.scale, dq[d][0], cur.x);
    cur.y = fmaf(a.scale, dq[d][1], cur.y);
    cur.z = fmaf(a.scale, dq[d][2], cur.z);
    cur.w = fmaf(a.scale, dq[d][3], cur.w);
    *(float4*)(dqp + 16 * d) = cur;
  }
}

// ---- dK, dV ---------------------------------------------------------------------------
template <int DQK, int DV>
struct F32DkvCfg {
  static constexpr int NK = 2, NQS = 4;               // 16-key blocks x query streams
  static constexpr int BKEY = 16 * NK, BQ = 16 * NQS; // keys per tile, query rows per query tile
  static constexpr int QS = DQK + 4, OS = DV + 4;
  static constexpr int Q_TILE = padded_tile_bytes(BQ, QS * 4) / 4;
  static constexpr int O_TILE = padded_tile_bytes(BQ, OS * 4) / 4;
  static constexpr int BUF = Q_TILE + O_TILE + 2 * BQ;   // Q, dO, LSE (log2 units), delta
  static constexpr int KT = DQK / 16, VT = DV / 16;      // dK, dV output tiles of 16 columns
  static constexpr int MERGE = 16 * (DQK + DV);          // one wave's dK, dV partial sums
  static_assert(NK * NQS == 8, "eight waves");
  static_assert(BQ == 64, "one wave loads a query tile's LSE and delta, one row per lane");
  static_assert(2 * BUF * 4 <= 160 * 1024, "LDS");
  static_assert((NQS - 1) * NK * MERGE <= 2 * BUF, "merge area");
};

// Key tile kt (BKEY keys) of one (batch, KV head): its dK, dV summed over the group's
// query heads and the query tiles that see it, added into the accumulators.
template <int DQK, int DV>
__device__ __forceinline__ void dkdv_f32_tile(const BwdArgs& a, int b, int kvg, int kt, float* smem) {
  using C = F32DkvCfg<DQK, DV>;
  constexpr int NK = C::NK, NQS = C::NQS, BKEY = C::BKEY, BQ = C::BQ, QS = C::QS, OS = C::OS;
  constexpr int KT = C::KT, VT = C::VT;
  const int lane = threadIdx.x & 63, lm = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int kblk = wave % NK, qs = wave / NK;
  const int key_base = kt * BKEY;
  int q_first = 0;   // the first query that can see the tile's first key
  if (a.causal) {
    const long long f = a.k_pos0 + key_base - a.q_pos0;
    q_first = (int)max(0LL, min(f, (long long)a.Sq));
  }
  if (q_first >= a.Sq) return;   // no query of the block sees these keys (workgroup-uniform)
  const int nqt = (a.Sq - q_first + BQ - 1) / BQ;
  const int ntiles = a.group * nqt;   // (query head of the group, query tile) pairs

  // stationary K and V of key lm of this wave's block (zero past the block)
  const int key = key_base + 16 * kblk + lm;
  const bool key_ok = key < a.Sk;
  const size_t kvh = (size_t)(b * a.Hkv + kvg) * a.Sk;
  float kreg[DQK / 4], vreg[DV / 4];
  load_vec(kreg, (const float*)a.k + (kvh + key) * DQK + g * (DQK / 4), key_ok);
  load_vec(vreg, (const float*)a.v + (kvh + key) * DV + g * (DV / 4), key_ok);
  const long long kpos = a.k_pos0 + key;
  const long long wk0 = a.k_pos0 + key_base + 16 * kblk;   // the wave's first key position
  f32x4 dk[KT], dv[VT];
#pragma unroll
  for (int t = 0; t < KT; ++t) dk[t] = f32x4{};
#pragma unroll
  for (int t = 0; t < VT; ++t) dv[t] = f32x4{};

  PaddedTileDma<BQ, DQK * 4, QS * 4, 8> qpad;
  PaddedTileDma<BQ, DV * 4, OS * 4, 8> opad;
  qpad.init(wave, lane);
  opad.init(wave, lane);
  const unsigned q_last = (unsigned)((size_t)a.Sq * DQK * 4 - 16), o_last = (unsigned)((size_t)a.Sq * DV * 4 - 16);
  auto tile_rows = [&](int n, int& bh, int& r0) __attribute__((always_inline)) {
    const int hh = n / nqt;
    bh = b * a.Hq + kvg * a.group + hh;
    r0 = q_first + (n - hh * nqt) * BQ;
  };
  auto dma = [&](int n, int buf) __attribute__((always_inline)) {
    int bh, r0;
    tile_rows(n, bh, r0);
    float* base = smem + buf * C::BUF;
    qpad.issue(wave, lds_addr(base), (unsigned)r0 * (DQK * 4), q_last,
               raw_desc((const float*)a.q + (size_t)bh * a.Sq * DQK, (unsigned)((size_t)a.Sq * DQK * 4)));
    opad.issue(wave, lds_addr(base + C::Q_TILE), (unsigned)r0 * (DV * 4), o_last,
               raw_desc((const float*)a.dout + (size_t)bh * a.Sq * DV, (unsigned)((size_t)a.Sq * DV * 4)));
  };
  // LSE (log2 units; +inf past the block or for a row with no visible key, so P = 0)
  // and delta of the tile's rows: wave 0, one row per lane
  auto stats = [&](int n, float& l2, float& dl) __attribute__((always_inline)) {
    int bh, r0;
    tile_rows(n, bh, r0);
    const int r = r0 + lane;
    l2 = __builtin_huge_valf();
    dl = 0.f;
    if (r < a.Sq) {
      const float l = a.lse[(size_t)bh * a.Sq + r];
      if (l != kNegInf) l2 = l * kLog2e;
      dl = a.delta[(size_t)bh * a.Sq + r];
    }
  };
  auto put_stats = [&](int buf, float l2, float dl) __attribute__((always_inline)) {
    float* st = smem + buf * C::BUF + C::Q_TILE + C::O_TILE;
    st[lane] = l2;
    st[BQ + lane] = dl;
  };

  __syncthreads();   // the previous key tile's buffers and partial sums are consumed
  dma(0, 0);
  if (wave == 0) {
    float l2, dl;
    stats(0, l2, dl);
    put_stats(0, l2, dl);
  }
  wait_vmem();
  __syncthreads();
  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    float l2n = 0.f, dln = 0.f;
    if (n + 1 < ntiles) {
      dma(n + 1, buf ^ 1);
      if (wave == 0) stats(n + 1, l2n, dln);
    }
    int bh, r0;
    tile_rows(n, bh, r0);
    const int rs = 16 * qs;                          // this stream's rows of the tile
    const long long qp0 = a.q_pos0 + r0 + rs;        // their first position
    bool skip = r0 + rs >= a.Sq;
    if (a.causal) skip = skip || qp0 + 15 < wk0;
    const bool need_mask = a.causal && qp0 < wk0 + 15;
    if (!skip) {
      const float* base = smem + buf * C::BUF;
      const float* qt = base;
      const float* ot = base + C::Q_TILE;
      const float* st = base + C::Q_TILE + C::O_TILE;
      // S and dP: lane holds key lm against rows rs + 4 g + v
      const f32x4 s = chain(qt + (rs + lm) * QS + g * (DQK / 4), kreg, f32x4{});
      const f32x4 dp = chain(ot + (rs + lm) * OS + g * (DV / 4), vreg, f32x4{});
      const float4 l4 = *(const float4*)(st + rs + 4 * g);
      const float4 d4 = *(const float4*)(st + BQ + rs + 4 * g);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
      float p[4], ds[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool vis = !need_mask || kpos <= qp0 + 4 * g + v;
        p[v] = vis ? exp2_hw(fmaf(s[v], a.scale_log2, -lv[v])) : 0.f;
        ds[v] = p[v] * (dp[v] - dv4[v]);
      }
      // dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS: product t takes row rs + 4 g + t
      const float* oc = ot + (rs + 4 * g) * OS + lm;
      const float* qc = qt + (rs + 4 * g) * QS + lm;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int d = 0; d < VT; ++d) dv[d] = mma16_f32(oc[t * OS + 16 * d], p[t], dv[d]);
#pragma unroll
        for (int d = 0; d < KT; ++d) dk[d] = mma16_f32(qc[t * QS + 16 * d], ds[t], dk[d]);
      }
    }
    if (wave == 0 && n + 1 < ntiles) put_stats(buf ^ 1, l2n, dln);
    wait_vmem();   // this wave's loads of tile n + 1 have landed
    __syncthreads();
  }

  // the query streams' sums meet in LDS (the tile buffers are free after the last barrier)
  if (qs > 0) {
    float* mb = smem + ((qs - 1) * NK + kblk) * C::MERGE;
#pragma unroll
    for (int d = 0; d < KT; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) mb[(4 * d + v) * 64 + lane] = dk[d][v];
#pragma unroll
    for (int d = 0; d < VT; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) mb[(4 * (KT + d) + v) * 64 + lane] = dv[d][v];
  }
  __syncthreads();
  if (qs > 0 || !key_ok) return;
#pragma unroll
  for (int s2 = 1; s2 < NQS; ++s2) {
    const float* mb = smem + ((s2 - 1) * NK + kblk) * C::MERGE;
#pragma unroll
    for (int d = 0; d < KT; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) dk[d][v] += mb[(4 * d + v) * 64 + lane];
#pragma unroll
    for (int d = 0; d < VT; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) dv[d][v] += mb[(4 * (KT + d) + v) * 64 + lane];
  }
  float* dkp = a.dk + (kvh + key) * DQK + 4 * g;
#pragma unroll
  for (int d = 0; d < KT; ++d) {
    float4 cur = *(const float4*)(dkp + 16 * d);
    cur.x = fmaf(a.scale, dk[d][0], cur.x);
    cur.y = fmaf(a.scale, dk[d][1], cur.y);
    cur.z = fmaf(a.scale, dk[d][2], cur.z);
    cur.w = fmaf(a.scale, dk[d][3], cur.w);
    *(float4*)(dkp + 16 * d) = cur;
  }
  float* dvp = a.dv + (kvh + key) * DV + 4 * g;
#pragma unroll
  for (int d = 0; d < VT; ++d) {
    float4 cur = *(const float4*)(dvp + 16 * d);
    cur.x += dv[d][0];
    cur.y += dv[d][1];
    cur.z += dv[d][2];
    cur.w += dv[d][3];
    *(float4*)(dvp + 16 * d) = cur;
  }
}

// Under a causal mask a workgroup takes key tiles kt and n - 1 - kt of one (batch,
// KV head), one after the other: the first sees about as many query tiles as the
// second misses, so every workgroup has about the same work; with fewer workgroups
// than the chip holds at once, an unpaired grid would last as long as its first
// (heaviest) tile. Without a mask every tile has the same work and a workgroup
// takes one.
template <int DQK, int DV>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_f32_kernel(BwdArgs a) {
  using C = F32DkvCfg<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) float smem[2 * C::BUF];
  const int nkt = (a.Sk + C::BKEY - 1) / C::BKEY;
  const int kt = (int)(blockIdx.x % a.n_tiles);   // a.n_tiles: ceil(nkt / 2) causal, nkt otherwise
  const int bg = blockIdx.x / a.n_tiles;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  dkdv_f32_tile<DQK, DV>(a, b, g, kt, smem);
  if (a.causal && nkt - 1 - kt != kt) dkdv_f32_tile<DQK, DV>(a, b, g, nkt - 1 - kt, smem);
}

// ---- launchers ------------------------------------------------------------------------
hipError_t bwd_delta_f32(const float* o, const float* dout, float* delta, long long rows, int Dv, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long long grid = (rows + 15) / 16;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_delta_f32_kernel, dim3((unsigned)grid), dim3(256), 0, st, o, dout, delta, rows, Dv);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t bwd_f32_launch(BwdArgs a, hipStream_t st) {
  using CK = F32DkvCfg<DQK, DV>;
  using CQ = F32DqCfg<DQK, DV, 4>;
  BwdArgs b = a;
  const int nkt = (a.Sk + CK::BKEY - 1) / CK::BKEY;
  b.n_tiles = a.causal ? (nkt + 1) / 2 : nkt;   // causal: pairs of key tiles
  long long grid = (long long)a.B * a.Hkv * b.n_tiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid > 0) hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DQK, DV>), dim3((unsigned)grid), dim3(512), 0, st, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 64-row dQ workgroups (4 row blocks x 2 key streams), or 32-row ones (2 x 4) when
  // there are fewer 64-row workgroups than CUs (measured on one head of 1024 rows:
  // 86 against 112 us for the whole step; slightly slower on large launches)
  const bool wide = (long long)a.B * a.Hq * ((a.Sq + CQ::BQ - 1) / CQ::BQ) >= 256;
  const int bq = wide ? CQ::BQ : CQ::BQ / 2;
  b.n_tiles = (a.Sq + bq - 1) / bq;
  grid = (long long)a.B * a.Hq * b.n_tiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid > 0) {
    if (wide)
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DQK, DV, 4>), dim3((unsigned)grid), dim3(512), 0, st, b);
    else
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DQK, DV, 2>), dim3((unsigned)grid), dim3(512), 0, st, b);
  }
  return hipGetLastError();
}

// Returns hipErrorInvalidValue when no kernel instance covers (dqk, dv).
hipError_t bwd_f32(const BwdArgs& a, int dqk, int dv, hipStream_t st) {
  if (dqk == 64 && dv == 64) return bwd_f32_launch<64, 64>(a, st);
  if (dqk == 64 && dv == 128) return bwd_f32_launch<64, 128>(a, st);
  if (dqk == 128 && dv == 64) return bwd_f32_launch<128, 64>(a, st);
  if (dqk == 128 && dv == 128) return bwd_f32_launch<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
