// fp32 blockwise exact attention (ring prefill and single ring step) for gfx950.
//
// Same protocol as the bf16 kernel: every KV tile updates the per-row running
// maximum and exp-sum, rescales the output accumulator and adds the tile's
// contribution (page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条
// 超长序列", §"最容易被忽略的细节"; blocks in the ring order of §"KV 在 Ring 中如何
// 流动"). Everything stays in fp32 (no bf16 rounding anywhere), on the vector ALUs:
// this path exists for fp32 inputs, whose tolerance no bf16 matrix-core product
// could meet.
//
// A workgroup owns 16 R query rows (R = 1, or 2 for launches of at least 1024
// 16-row tiles) and walks the keys in tiles of 64 (32 when D_qk + D_v > 128),
// split over NS groups of 256 threads ("key streams": 4 for R = 1; for R = 2, 3 at
// D = 64 and 2 at D = 128), each taking every NS-th tile. Thread t of a group
// works for rows t / 16 + 16 r, r < R (the 16 threads of a row group sit in one
// wave):
//   score phase: keys (t % 16) + 16 u, u < BK / 16; each step reads four
//                consecutive d of the rows' queries (broadcast 16-byte LDS reads
//                of padded rows) and of each of its keys (16-byte reads of padded
//                K rows, conflict-free), then 4 R FMAs per key;
//   PV phase:    output columns 4 (t % 16) .. + 3 (and + 64 when D_v = 128); each
//                step reads four probabilities of each row (broadcast) and, per
//                key, four consecutive V values (16-byte reads), then 4 R FMAs per
//                key and column group.
// The row's 16 threads exchange the tile's max and sum with xor-shuffles inside
// their group of 16 lanes. The next K/V tile is fetched into registers while the
// current one is computed. At the end the groups' states are merged in LDS. Several
// streams keep 8 to 16 waves on a CU where one 256-thread workgroup with
// double-buffered tiles (145 KB at D = 128) kept 4, and they split a small
// launch's key range over more waves; two rows per thread halve the K and V reads
// per FMA where the launch has the workgroups to spare.
#include "common.hpp"

namespace ra {

enum { F32_RING = 0, F32_STEP = 1 };

template <int DQK, int DV>
struct F32Cfg {
  // 64-key tiles at D_qk = D_v = 64, 32-key tiles otherwise (measured: at D = 64,
  // 32-key tiles are 10-15 % slower and 128-key tiles 25 % slower; at D = 128,
  // 32-key tiles are 1.5x faster: half the LDS and 50 fewer registers per thread)
  static constexpr int BQ = 16, BK = DQK + DV <= 128 ? 64 : 32, THREADS = 256;
  static constexpr int KPT = BK / 16;  // keys per thread in the score phase
  static constexpr int KS = DQK + 4;   // padded K rows: 16 consecutive rows start on 16 distinct 4-bank groups
  static constexpr int QS = DQK + 4;   // padded Q rows: a wave's four rows start on distinct 4-bank groups
  static constexpr int PS = BK + 4;
  static constexpr int NV = DV / 64;   // float4 output groups per thread
  static constexpr int KCH = BK * DQK / 4 / THREADS;   // float4 K loads per thread per tile
  static constexpr int VCH = BK * DV / 4 / THREADS;    // float4 V loads per thread per tile
  static_assert(KCH * THREADS * 4 == BK * DQK && VCH * THREADS * 4 == BK * DV, "tile split");
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
    bh = blockIdx.x / tiles_per_head;
    const int gt = tiles_per_head - 1 - (int)(blockIdx.x % tiles_per_head);
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

// NS groups of 256 threads ("key streams") share one query tile: group s takes key
// tiles s, s + NS, s + 2 NS, ... (single-buffered LDS, the next tile prefetched in
// registers), and the groups' running states (m, l, O) meet in LDS at the end: with
// M the largest m, l = sum l_s 2^(m_s - M) and O = sum O_s 2^(m_s - M), the merge of
// partial softmax states over disjoint key sets.
template <int DQK, int DV, int NS_, int R_>
struct F32StreamCfg {
  using C = F32Cfg<DQK, DV>;
  static constexpr int NS = NS_, R = R_;
  static constexpr int BQ = 16 * R;                      // query rows per workgroup
  static constexpr int KV = C::BK * C::KS + C::BK * DV;  // one stream's K and V tile
  static_assert(BQ * DV <= KV, "a stream's partial output fits its K / V area");
  static_assert((BQ * C::QS + NS * (KV + BQ * C::PS)) * 4 <= 160 * 1024, "LDS");
};

// R rows per thread: the 16 threads of row group qi serve rows qi + 16 r, r < R, so
// every K (V) chunk read from LDS feeds R rows.
template <int DQK, int DV, int MODE, int NS_, int R_>
__global__ void __launch_bounds__(NS_ * 256)
prefill_f32_kernel(PrefillArgs a) {
  using C = F32Cfg<DQK, DV>;
  using SC = F32StreamCfg<DQK, DV, NS_, R_>;
  constexpr int BK = C::BK, KS = C::KS, QS = C::QS, PS = C::PS, NV = C::NV, NS = SC::NS, R = SC::R;
  constexpr int BQ = SC::BQ, KPT = C::KPT;
  constexpr int T = C::THREADS;
  __shared__ __attribute__((aligned(16))) float qsm[BQ * QS];
  __shared__ __attribute__((aligned(16))) float kvsm[NS][SC::KV];
  __shared__ __attribute__((aligned(16))) float psm[NS][BQ * PS];

  const int tid = threadIdx.x, st = tid / T, lt = tid % T;
  const int qi = lt >> 4;   // row group: rows qi + 16 r of the tile
  const int j = lt & 15;
  float* ksm = kvsm[st];
  float* vsm = kvsm[st] + BK * KS;
  float* prow = psm[st];

  F32Work<BQ, BK, MODE> w;
  if (!w.init(a)) return;
  const int bh = w.bh, row_base = w.row_base, row_end = w.row_end, ntiles = w.ntiles;
  const float* q_head = (const float*)a.q + (size_t)bh * a.q_rows * DQK;
  const float* k_head = (const float*)a.k + w.kvh * DQK;
  const float* v_head = (const float*)a.v + w.kvh * DV;

  for (int e = tid; e < BQ * DQK / 4; e += NS * T) {
    const int r = e / (DQK / 4), c4 = e % (DQK / 4);
    const int row = row_base + r;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < row_end) x = *(const float4*)(q_head + (size_t)row * DQK + 4 * c4);
    *(float4*)&qsm[r * QS + 4 * c4] = x;
  }

  float4 kr[C::KCH], vr[C::VCH];
  auto load_tile = [&](int krow0, int nvalid) {
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      const int e = it * T + lt, r = e / (DQK / 4), c4 = e % (DQK / 4);
      kr[it] = r < nvalid ? *(const float4*)(k_head + (size_t)(krow0 + r) * DQK + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < C::VCH; ++it) {
      const int e = it * T + lt, r = e / (DV / 4), c4 = e % (DV / 4);
      vr[it] = r < nvalid ? *(const float4*)(v_head + (size_t)(krow0 + r) * DV + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      const int e = it * T + lt, r = e / (DQK / 4), c4 = e % (DQK / 4);
      *(float4*)&ksm[r * KS + 4 * c4] = kr[it];
    }
#pragma unroll
    for (int it = 0; it < C::VCH; ++it) {
      const int e = it * T + lt, r = e / (DV / 4), c4 = e % (DV / 4);
      *(float4*)&vsm[r * DV + 4 * c4] = vr[it];
    }
  };

  float4 acc[R][NV];
  float m[R], l[R];
  long long my_pos[R];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
    my_pos[h] = w.pos_base + qi + 16 * h;
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[h][e] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int my_row = row_base + qi + 16 * h;
    if (MODE == F32_STEP && st == 0 && my_row < row_end) {
      // the running state enters through the first stream
      const size_t r = (size_t)bh * a.q_rows + my_row;
      const float lin = a.lse_acc[r];
      if (lin != kNegInf) {
        m[h] = lin * kLog2e;
        l[h] = 1.f;
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[h][e] = *(const float4*)(a.o_acc + r * DV + 64 * e + 4 * j);
      }
    }
  }

  int krow0 = 0, nvalid = 0;
  long long kpos0 = 0;
  if (st < ntiles) {
    w.tile_at(st, krow0, kpos0, nvalid);
    load_tile(krow0, nvalid);
  }
  const int niter = (ntiles + NS - 1) / NS;
  for (int it = 0; it < niter; ++it) {
    const int n = it * NS + st;
    const bool active = n < ntiles;   // a stream past the end idles through the barriers
    const long long kpos_cur = kpos0;
    const int nvalid_cur = nvalid;
    __syncthreads();   // the previous tile is consumed (and Q is in LDS)
    if (active) store_tile();
    __syncthreads();   // this tile is in LDS
    if (n + NS < ntiles) {
      w.tile_at(n + NS, krow0, kpos0, nvalid);
      load_tile(krow0, nvalid);   // lands while this tile is computed
    }
    float alpha[R];
#pragma unroll
    for (int h = 0; h < R; ++h) alpha[h] = 1.f;
    if (active) {
      float s[R][KPT];
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int u = 0; u < KPT; ++u) s[h][u] = 0.f;
#pragma unroll 4
      for (int d4 = 0; d4 < DQK / 4; ++d4) {
        float4 qv[R];
#pragma unroll
        for (int h = 0; h < R; ++h) qv[h] = *(const float4*)&qsm[(qi + 16 * h) * QS + 4 * d4];
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
          const float4 kv = *(const float4*)&ksm[(j + 16 * u) * KS + 4 * d4];
#pragma unroll
          for (int h = 0; h < R; ++h) {
            s[h][u] = fmaf(qv[h].x, kv.x, s[h][u]);
            s[h][u] = fmaf(qv[h].y, kv.y, s[h][u]);
            s[h][u] = fmaf(qv[h].z, kv.z, s[h][u]);
            s[h][u] = fmaf(qv[h].w, kv.w, s[h][u]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < R; ++h) {
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
          const int key = j + 16 * u;
          const bool ok = key < nvalid_cur && (!a.causal || kpos_cur + key <= my_pos[h]);
          s[h][u] = ok ? s[h][u] : kNegInf;
          mx = fmaxf(mx, s[h][u]);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
        const float mnew = fmaxf(m[h], mx * a.scale_log2);
        const float muse = mnew == kNegInf ? 0.f : mnew;
        alpha[h] = exp2_hw(m[h] - muse);
        m[h] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
          const float p = exp2_hw(fmaf(s[h][u], a.scale_log2, -muse));
          prow[(qi + 16 * h) * PS + j + 16 * u] = p;
          rs += p;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) rs += shfl_xor_f(rs, o);
        l[h] = l[h] * alpha[h] + rs;
      }
    }
    __syncthreads();   // the rows' probabilities are in LDS
    if (active) {
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          acc[h][e].x *= alpha[h];
          acc[h][e].y *= alpha[h];
          acc[h][e].z *= alpha[h];
          acc[h][e].w *= alpha[h];
        }
#pragma unroll 2
      for (int c4 = 0; c4 < BK / 4; ++c4) {
        float pk[R][4];
#pragma unroll
        for (int h = 0; h < R; ++h) {
          const float4 pv = *(const float4*)&prow[(qi + 16 * h) * PS + 4 * c4];
          pk[h][0] = pv.x;
          pk[h][1] = pv.y;
          pk[h][2] = pv.z;
          pk[h][3] = pv.w;
        }
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
#pragma unroll
          for (int e = 0; e < NV; ++e) {
            const float4 vv = *(const float4*)&vsm[(4 * c4 + e4) * DV + 64 * e + 4 * j];
#pragma unroll
            for (int h = 0; h < R; ++h) {
              acc[h][e].x = fmaf(pk[h][e4], vv.x, acc[h][e].x);
              acc[h][e].y = fmaf(pk[h][e4], vv.y, acc[h][e].y);
              acc[h][e].z = fmaf(pk[h][e4], vv.z, acc[h][e].z);
              acc[h][e].w = fmaf(pk[h][e4], vv.w, acc[h][e].w);
            }
          }
        }
      }
    }
  }

  // merge: streams 1.. leave (m, l, O) in their own LDS areas, stream 0 combines
  __syncthreads();   // every tile is consumed
  if (st > 0) {
    float* ob = kvsm[st];
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const int row = qi + 16 * h;
#pragma unroll
      for (int e = 0; e < NV; ++e) *(float4*)&ob[row * DV + 64 * e + 4 * j] = acc[h][e];
      if (j == 0) {
        psm[st][2 * row] = m[h];
        psm[st][2 * row + 1] = l[h];
      }
    }
  }
  __syncthreads();
  if (st == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const int row = qi + 16 * h, my_row = row_base + row;
      if (my_row >= row_end) continue;
      float M = m[h];
#pragma unroll
      for (int t = 1; t < NS; ++t) M = fmaxf(M, psm[t][2 * row]);
      const float wown = m[h] == kNegInf ? 0.f : exp2_hw(m[h] - M);
      float lt_sum = l[h] * wown;
      float4 o4[NV];
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        o4[e].x = acc[h][e].x * wown;
        o4[e].y = acc[h][e].y * wown;
        o4[e].z = acc[h][e].z * wown;
        o4[e].w = acc[h][e].w * wown;
      }
#pragma unroll
      for (int t = 1; t < NS; ++t) {
        const float mt = psm[t][2 * row];
        const float wt = mt == kNegInf ? 0.f : exp2_hw(mt - M);
        lt_sum = fmaf(psm[t][2 * row + 1], wt, lt_sum);
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          const float4 o = *(const float4*)&kvsm[t][row * DV + 64 * e + 4 * j];
          o4[e].x = fmaf(o.x, wt, o4[e].x);
          o4[e].y = fmaf(o.y, wt, o4[e].y);
          o4[e].z = fmaf(o.z, wt, o4[e].z);
          o4[e].w = fmaf(o.w, wt, o4[e].w);
        }
      }
      const size_t r = (size_t)bh * a.q_rows + my_row;
      const float inv = lt_sum > 0.f ? 1.f / lt_sum : 0.f;
      const float lse = lt_sum > 0.f ? (M + log2_hw(lt_sum)) * kLn2 : kNegInf;
      float* out = MODE == F32_RING ? (float*)a.o : a.o_acc;
#pragma unroll
      for (int e = 0; e < NV; ++e)
        *(float4*)(out + r * DV + 64 * e + 4 * j) = make_float4(o4[e].x * inv, o4[e].y * inv, o4[e].z * inv,
                                                                o4[e].w * inv);
      if (j == 0) {
        if (MODE == F32_RING)
          a.lse[r] = lse;
        else
          a.lse_acc[r] = lse;
      }
    }
  }
}

template <int DQK, int DV, int MODE, int NS, int R>
static hipError_t launch_f32_as(PrefillArgs a, hipStream_t st) {
  const int rows_per_part = MODE == F32_RING ? a.Sp : a.q_rows;
  a.n_qtiles = (rows_per_part + 16 * R - 1) / (16 * R);
  const long long tiles = (long long)a.B * a.Hq * (MODE == F32_RING ? a.nq : 1) * a.n_qtiles;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_kernel<DQK, DV, MODE, NS, R>), dim3((unsigned)tiles), dim3(NS * 256), 0, st, a);
  return hipGetLastError();
}

template <int DQK, int DV, int MODE>
static hipError_t launch_f32(PrefillArgs a, hipStream_t st) {
  const int rows_per_part = MODE == F32_RING ? a.Sp : a.q_rows;
  const long long tiles16 = (long long)a.B * a.Hq * (MODE == F32_RING ? a.nq : 1) * ((rows_per_part + 15) / 16);
  // Launches of fewer than 1024 16-row tiles split each tile's keys over four
  // streams; larger ones (two or more 32-row workgroups per CU) take two rows per
  // thread with three streams at D = 64 and two at D = 128, what fits 160 KB of LDS.
  if (tiles16 < 1024) return launch_f32_as<DQK, DV, MODE, 4, 1>(a, st);
  if constexpr (DQK + DV <= 128)
    return launch_f32_as<DQK, DV, MODE, 3, 2>(a, st);
  else
    return launch_f32_as<DQK, DV, MODE, 2, 2>(a, st);
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
