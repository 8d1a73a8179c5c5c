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
// Workgroup: 256 threads, 32 query rows, key tiles of 32 staged in LDS.
//   score phase: thread t owns query t/8 and keys (t%8) + 8u, u = 0..3
//   PV phase:    thread t owns query t/8 and output columns (t%8) + 8e
// The eight threads of a query exchange the row max / sum with xor-shuffles.
#include "common.hpp"

namespace ra {

enum { F32_RING = 0, F32_STEP = 1 };

template <int DQK, int DV, int MODE>
__global__ void __launch_bounds__(256)
prefill_f32_kernel(PrefillArgs a) {
  constexpr int BQ = 32, BK = 32;
  constexpr int QS = DQK + 1;  // padded rows: conflict-free column walks
  constexpr int KS = DQK + 1;
  constexpr int PS = BK + 1;
  __shared__ float qs[BQ * QS];
  __shared__ float ksm[BK * KS];
  __shared__ float vsm[BK * DV];
  __shared__ float ps[BQ * PS];

  const int tid = threadIdx.x;
  const int qi = tid >> 3;   // query row inside the tile
  const int sub = tid & 7;

  const int tiles_per_head = (MODE == F32_RING ? a.nq : 1) * a.n_qtiles;
  const int bh = blockIdx.x / tiles_per_head;
  const int gt = tiles_per_head - 1 - (int)(blockIdx.x % tiles_per_head);
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int g = hq / a.group;
  int part = 0, qt = gt;
  if (MODE == F32_RING) {
    part = gt / a.n_qtiles;
    qt = gt - part * a.n_qtiles;
  }
  int row_base, row_end;
  long long pos_base;
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

  const float* q_head = (const float*)a.q + (size_t)bh * a.q_rows * DQK;
  const size_t kvh = (size_t)(b * a.Hkv + g) * a.kv_rows;
  const float* k_head = (const float*)a.k + kvh * DQK;
  const float* v_head = (const float*)a.v + kvh * DV;

  // tile schedule (the same RingTiles rules as the bf16 kernel)
  RingTiles ring;
  int ntiles;
  if (MODE == F32_RING) {
    ring.init(a.q_part0 + part, a.P, a.Sp, BK, a.causal != 0, a.striped != 0, last_row - part * a.Sp);
    ntiles = ring.ntiles;
  } else {
    long long kmax = a.Sk;
    if (a.causal) kmax = min(kmax, last_pos - a.k_pos0 + 1);
    if (kmax <= 0) return;
    ntiles = (int)((kmax + BK - 1) / BK);
  }

  // queries of the tile into LDS (zero past the end)
  for (int e = tid; e < BQ * DQK; e += 256) {
    const int r = e / DQK, d = e % DQK;
    const int row = row_base + r;
    qs[r * QS + d] = row < row_end ? q_head[(size_t)row * DQK + d] : 0.f;
  }

  const int my_row = row_base + qi;
  const long long my_pos = pos_base + qi;
  constexpr int NE = DV / 8;
  float acc[NE];
  float m = kNegInf, l = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.f;
  if (MODE == F32_STEP && my_row < row_end) {
    const size_t r = (size_t)bh * a.q_rows + my_row;
    const float lin = a.lse_acc[r];
    if (lin != kNegInf) {
      m = lin * kLog2e;
      l = 1.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] = a.o_acc[r * DV + sub + 8 * e];
    }
  }

  for (int n = 0; n < ntiles; ++n) {
    int krow0, nvalid;
    long long kpos0;
    if (MODE == F32_RING) {
      ring.tile(n, krow0, kpos0, nvalid);
    } else {
      krow0 = n * BK;
      kpos0 = a.k_pos0 + (long long)n * BK;
      nvalid = min(BK, a.Sk - n * BK);
    }
    __syncthreads();  // previous tile fully consumed (and Q staged on entry)
    for (int e = tid; e < BK * DQK; e += 256) {
      const int r = e / DQK, d = e % DQK;
      ksm[r * KS + d] = r < nvalid ? k_head[(size_t)(krow0 + r) * DQK + d] : 0.f;
    }
    for (int e = tid; e < BK * DV; e += 256) {
      const int r = e / DV, d = e % DV;
      vsm[r * DV + d] = r < nvalid ? v_head[(size_t)(krow0 + r) * DV + d] : 0.f;
    }
    __syncthreads();

    float s[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) s[u] = 0.f;
    for (int d = 0; d < DQK; ++d) {
      const float qv = qs[qi * QS + d];
#pragma unroll
      for (int u = 0; u < 4; ++u) s[u] = fmaf(qv, ksm[(sub + 8 * u) * KS + d], s[u]);
    }
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = sub + 8 * u;
      const bool ok = key < nvalid && (!a.causal || kpos0 + key <= my_pos);
      s[u] = ok ? s[u] : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 1));
    mx = fmaxf(mx, shfl_xor_f(mx, 2));
    mx = fmaxf(mx, shfl_xor_f(mx, 4));
    const float mnew = fmaxf(m, mx * a.scale_log2);
    const float muse = mnew == kNegInf ? 0.f : mnew;
    const float alpha = exp2_hw(m - muse);
    m = mnew;
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p = exp2_hw(fmaf(s[u], a.scale_log2, -muse));
      ps[qi * PS + sub + 8 * u] = p;
      rs += p;
    }
    rs += shfl_xor_f(rs, 1);
    rs += shfl_xor_f(rs, 2);
    rs += shfl_xor_f(rs, 4);
    l = l * alpha + rs;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] *= alpha;
    for (int k = 0; k < BK; ++k) {
      const float p = ps[qi * PS + k];
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] = fmaf(p, vsm[k * DV + sub + 8 * e], acc[e]);
    }
  }

  if (my_row < row_end) {
    const size_t r = (size_t)bh * a.q_rows + my_row;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? (m + log2_hw(l)) * kLn2 : kNegInf;
    float* out = MODE == F32_RING ? (float*)a.o : a.o_acc;
#pragma unroll
    for (int e = 0; e < NE; ++e) out[r * DV + sub + 8 * e] = acc[e] * inv;
    if (sub == 0) {
      if (MODE == F32_RING)
        a.lse[r] = lse;
      else
        a.lse_acc[r] = lse;
    }
  }
}

template <int DQK, int DV, int MODE>
static hipError_t launch_f32(PrefillArgs a, hipStream_t st) {
  const int rows_per_part = MODE == F32_RING ? a.Sp : a.q_rows;
  a.n_qtiles = (rows_per_part + 31) / 32;
  const long long tiles = (long long)a.B * a.Hq * (MODE == F32_RING ? a.nq : 1) * a.n_qtiles;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_kernel<DQK, DV, MODE>), dim3((unsigned)tiles), dim3(256), 0, st, a);
  return hipGetLastError();
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
