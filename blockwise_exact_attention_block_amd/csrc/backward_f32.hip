// Backward pass of blockwise exact attention for fp32 inputs on gfx950, on the
// vector ALUs.
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
// Three kernels:
//   * bwd_delta_f32_kernel: delta per query row, 16 lanes per row.
//   * bwd_dq_f32_kernel (256 threads): 32 query rows of one (batch, head) per
//     workgroup (16 in launches of fewer 32-row workgroups than CUs), key tiles of 64
//     (D_qk = D_v = 64) or 32 in LDS, the next tile prefetched into registers. Thread
//     t first forms S and dP for keys t % 16 + 16 u against rows t / 16 and
//     t / 16 + 16, then accumulates dQ for D_qk / 32 rows (half that with 16-row
//     workgroups) at one group of four columns, reading their dS (stored key-major)
//     as one vector.
//   * bwd_dkdv_f32_kernel (512 threads): key tiles of 32 of one (batch, KV head), the
//     tile's K and V rows in LDS; it walks the group's query heads and the visible
//     query tiles of 32 rows, the two halves of the workgroup taking alternate ones.
//     Thread t of a half first forms P and dS for keys t % 16, t % 16 + 16 against
//     rows t / 16, t / 16 + 16, then accumulates dK (dV) for D_qk / 32 (D_v / 32) keys
//     at one group of four columns, reading their dS (P) as one vector; the halves'
//     sums meet in LDS at the end. Under a causal mask a workgroup takes key tiles kt
//     and n - 1 - kt, which balances the work.
// Each thread works on two rows by two or more keys, so every 16-byte LDS read
// feeds 8 or more FMAs. LDS rows are padded by 4 floats; every sum runs in a fixed
// order, so results are reproducible run to run.
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

template <int DQK, int DV>
struct F32BCfg {
  static constexpr int THREADS = 256;
  static constexpr int BQK = 32;                // query rows per tile (both kernels)
  // keys per tile in the dQ kernel: 32 unless D_qk = D_v = 64, so that two
  // workgroups fit a CU's LDS
  static constexpr int BK = DQK + DV > 128 ? 32 : 64;
  static constexpr int NU = BK / 16;            // keys per thread in the dQ kernel's score pass
  static constexpr int BKEY = 32;               // keys per tile (dK/dV)
  // keys per thread in the dK (dV) sums; also rows per thread in the dQ sums
  static constexpr int KK = DQK / 32, KVV = DV / 32;
  // every LDS row padded by 4 floats: 16-byte reads of up to 16 rows at one column
  // start on distinct 4-bank groups
  static constexpr int QS = DQK + 4, OS = DV + 4, KS = DQK + 4, VS = DV + 4;
  static constexpr int PS2 = BKEY + 4;
  static constexpr int KCH = BK * DQK / 4 / THREADS, VCH = BK * DV / 4 / THREADS;
  static constexpr int QCH2 = BQK * DQK / 4 / THREADS, OCH2 = BQK * DV / 4 / THREADS;
  static_assert(KCH * THREADS * 4 == BK * DQK && VCH * THREADS * 4 == BK * DV, "tile split");
  static_assert(QCH2 * THREADS * 4 == BQK * DQK && OCH2 * THREADS * 4 == BQK * DV, "tile split");
  static_assert(DQK % 64 == 0 && DV % 64 == 0, "64-column groups");
};

__device__ __forceinline__ float dot4(float4 x, float4 y, float acc) {
  acc = fmaf(x.x, y.x, acc);
  acc = fmaf(x.y, y.y, acc);
  acc = fmaf(x.z, y.z, acc);
  return fmaf(x.w, y.w, acc);
}
__device__ __forceinline__ void axpy4(float s, float4 x, float4& acc) {
  acc.x = fmaf(s, x.x, acc.x);
  acc.y = fmaf(s, x.y, acc.y);
  acc.z = fmaf(s, x.z, acc.z);
  acc.w = fmaf(s, x.w, acc.w);
}
__device__ __forceinline__ float4 lds4(const float* p) { return *(const float4*)p; }

// Rows [row0, row0 + rows) of a [n, D] fp32 matrix, 16-byte chunks dealt round-robin
// over the workgroup's threads (chunk e = it * THREADS + tid); rows at or past
// `limit` read as zero.
template <int D, int CH, int THREADS>
__device__ __forceinline__ void load_rows(float4 (&r)[CH], const float* base, int row0, int limit, int tid) {
#pragma unroll
  for (int it = 0; it < CH; ++it) {
    const int e = it * THREADS + tid, rr = e / (D / 4), c4 = e % (D / 4);
    r[it] = row0 + rr < limit ? *(const float4*)(base + (size_t)(row0 + rr) * D + 4 * c4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}
template <int D, int CH, int THREADS, int STRIDE>
__device__ __forceinline__ void store_rows(const float4 (&r)[CH], float* lds, int tid) {
#pragma unroll
  for (int it = 0; it < CH; ++it) {
    const int e = it * THREADS + tid, rr = e / (D / 4), c4 = e % (D / 4);
    *(float4*)&lds[rr * STRIDE + 4 * c4] = r[it];
  }
}

template <int N>
__device__ __forceinline__ void lds_n(float (&x)[N], const float* p) {
  if constexpr (N == 4) {
    const float4 v = *(const float4*)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else if constexpr (N == 2) {
    const float2 v = *(const float2*)p;
    x[0] = v.x; x[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
  }
}

// ---- dQ -------------------------------------------------------------------------------
// 16 R query rows of one (batch, head) per workgroup (R = 2, or 1 for launches of
// fewer 32-row workgroups than CUs). Score pass: keys kp + 16 u (u < BK / 16)
// against rows rq + 16 h, h < R (kp = t % 16, rq = t / 16), each K / V chunk read
// once for the R rows and each Q / dO chunk once for all the keys; dS goes to LDS
// key-major. dQ pass: rows RQ (t / (DQK/4)) .. + RQ - 1 at columns
// 4 (t % (DQK/4)) .. + 3, one vector read of their dS and one of K per key.
template <int DQK, int DV, int R>
__global__ void __launch_bounds__(256)
bwd_dq_f32_kernel(BwdArgs a) {
  using C = F32BCfg<DQK, DV>;
  constexpr int BQ = 16 * R, BK = C::BK, NU = C::NU, QS = C::QS, OS = C::OS, KS = C::KS, VS = C::VS;
  constexpr int T = C::THREADS, RQ = BQ * DQK / 4 / T, DSS = BQ + 4;
  constexpr int QCH = BQ * DQK / 4 / T, OCH = BQ * DV / 4 / T;
  static_assert(RQ * T * 4 == BQ * DQK && QCH * T * 4 == BQ * DQK && OCH * T * 4 == BQ * DV, "tile split");
  __shared__ __attribute__((aligned(16))) float qsm[BQ * QS];
  __shared__ __attribute__((aligned(16))) float osm[BQ * OS];
  __shared__ __attribute__((aligned(16))) float ksm[BK * KS];
  __shared__ __attribute__((aligned(16))) float vsm[BK * VS];
  __shared__ __attribute__((aligned(16))) float dst[BK * DSS];   // dS, key-major

  const int tid = threadIdx.x, kp = tid & 15, rq = tid >> 4;
  const int cg = tid % (DQK / 4), rg = tid / (DQK / 4);
  // workgroup -> (batch, head, query tile), the heaviest causal tiles first
  const int qt = a.n_tiles - 1 - (int)(blockIdx.x % a.n_tiles);
  const int bh = blockIdx.x / a.n_tiles;
  const int b = bh / a.Hq, hq = bh - b * a.Hq, g = hq / a.group;
  const int row_base = qt * BQ;
  const int last_row = min(row_base + BQ, a.Sq) - 1;
  long long kmax = a.Sk;
  if (a.causal) kmax = min(kmax, a.q_pos0 + last_row - a.k_pos0 + 1);
  if (kmax <= 0) return;   // no key of the block is visible to this tile
  const int ntiles = (int)((kmax + BK - 1) / BK);

  const float* q_head = (const float*)a.q + (size_t)bh * a.Sq * DQK;
  const float* o_head = (const float*)a.dout + (size_t)bh * a.Sq * DV;
  const size_t kvh = (size_t)(b * a.Hkv + g) * a.Sk;
  const float* k_head = (const float*)a.k + kvh * DQK;
  const float* v_head = (const float*)a.v + kvh * DV;

  {
    float4 qr[QCH], orr[OCH];
    load_rows<DQK, QCH, T>(qr, q_head, row_base, a.Sq, tid);
    load_rows<DV, OCH, T>(orr, o_head, row_base, a.Sq, tid);
    store_rows<DQK, QCH, T, QS>(qr, qsm, tid);
    store_rows<DV, OCH, T, OS>(orr, osm, tid);
  }
  // statistics of rows rq + 16 h: a row past the block, or with no visible key, gets
  // P = 0
  float lse2[R], dlt[R];
  long long qpos[R];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const int row = row_base + rq + 16 * h;
    qpos[h] = a.q_pos0 + row;
    lse2[h] = __builtin_huge_valf();   // +inf: exp2(s - lse2) = 0
    dlt[h] = 0.f;
    if (row < a.Sq) {
      const float l = a.lse[(size_t)bh * a.Sq + row];
      if (l != kNegInf) lse2[h] = l * kLog2e;
      dlt[h] = a.delta[(size_t)bh * a.Sq + row];
    }
  }

  // K / V tiles: global -> registers (one tile ahead) -> LDS
  float4 kr[C::KCH], vr[C::VCH];
  float4 acc[RQ];
#pragma unroll
  for (int e = 0; e < RQ; ++e) acc[e] = make_float4(0.f, 0.f, 0.f, 0.f);

  load_rows<DQK, C::KCH, T>(kr, k_head, 0, a.Sk, tid);
  load_rows<DV, C::VCH, T>(vr, v_head, 0, a.Sk, tid);
  store_rows<DQK, C::KCH, T, KS>(kr, ksm, tid);
  store_rows<DV, C::VCH, T, VS>(vr, vsm, tid);
  __syncthreads();   // Q, dO and the first K / V tile are in LDS
  for (int n = 0; n < ntiles; ++n) {
    const long long kpos0 = a.k_pos0 + (long long)n * BK;
    const int nvalid = min(BK, a.Sk - n * BK);
    if (n + 1 < ntiles) {   // lands while this tile is computed
      load_rows<DQK, C::KCH, T>(kr, k_head, (n + 1) * BK, a.Sk, tid);
      load_rows<DV, C::VCH, T>(vr, v_head, (n + 1) * BK, a.Sk, tid);
    }
    float s[R][NU], dp[R][NU];
#pragma unroll
    for (int h = 0; h < R; ++h)
#pragma unroll
      for (int u = 0; u < NU; ++u) s[h][u] = dp[h][u] = 0.f;
#pragma unroll 2
    for (int d4 = 0; d4 < DQK / 4; ++d4) {
      float4 x[R];
#pragma unroll
      for (int h = 0; h < R; ++h) x[h] = lds4(&qsm[(rq + 16 * h) * QS + 4 * d4]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float4 kx = lds4(&ksm[(kp + 16 * u) * KS + 4 * d4]);
#pragma unroll
        for (int h = 0; h < R; ++h) s[h][u] = dot4(x[h], kx, s[h][u]);
      }
    }
#pragma unroll 2
    for (int d4 = 0; d4 < DV / 4; ++d4) {
      float4 x[R];
#pragma unroll
      for (int h = 0; h < R; ++h) x[h] = lds4(&osm[(rq + 16 * h) * OS + 4 * d4]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float4 vx = lds4(&vsm[(kp + 16 * u) * VS + 4 * d4]);
#pragma unroll
        for (int h = 0; h < R; ++h) dp[h][u] = dot4(x[h], vx, dp[h][u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int key = kp + 16 * u;
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const bool vis = key < nvalid && (!a.causal || kpos0 + key <= qpos[h]);
        const float p = vis ? exp2_hw(fmaf(s[h][u], a.scale_log2, -lse2[h])) : 0.f;
        dst[key * DSS + rq + 16 * h] = p * (dp[h][u] - dlt[h]);
      }
    }
    __syncthreads();   // the tile's dS is in LDS
    // dQ rows RQ rg .. + RQ - 1, columns 4 cg .. + 3, over the tile's keys
#pragma unroll 4
    for (int kk = 0; kk < BK; ++kk) {
      float ds[RQ];
      lds_n<RQ>(ds, &dst[kk * DSS + RQ * rg]);
      const float4 kx = lds4(&ksm[kk * KS + 4 * cg]);
#pragma unroll
      for (int e = 0; e < RQ; ++e) axpy4(ds[e], kx, acc[e]);
    }
    __syncthreads();   // K, V and dS of this tile consumed
    if (n + 1 < ntiles) {
      store_rows<DQK, C::KCH, T, KS>(kr, ksm, tid);
      store_rows<DV, C::VCH, T, VS>(vr, vsm, tid);
      __syncthreads();
    }
  }

#pragma unroll
  for (int e = 0; e < RQ; ++e) {
    const int row = row_base + RQ * rg + e;
    if (row < a.Sq) {
      float* dqp = a.dq + ((size_t)bh * a.Sq + row) * DQK + 4 * cg;
      float4 cur = *(const float4*)dqp;
      axpy4(a.scale, acc[e], cur);
      *(float4*)dqp = cur;
    }
  }
}

// ---- dK, dV ---------------------------------------------------------------------------
// One 32-key tile of one (batch, KV head): dK, dV of its keys summed over the group's
// query heads and the query tiles (32 rows) that see them, added into the
// accumulators. The workgroup's two halves of 256 threads walk alternate (head,
// query tile) pairs, each with its own Q / dO / P / dS tiles, and add their sums
// through LDS at the end.
template <int DQK, int DV>
struct F32KvSmem {
  using C = F32BCfg<DQK, DV>;
  // K and V rows; at the end, the second half's partial sums
  float kv[C::BKEY * (C::KS + C::VS)];
  float q[2][C::BQK * C::QS];
  float o[2][C::BQK * C::OS];
  float p[2][C::BQK * C::PS2];
  float ds[2][C::BQK * C::PS2];
  float l2[2][C::BQK];
  float dl[2][C::BQK];
};

template <int DQK, int DV>
__device__ __forceinline__ void dkdv_f32_tile(const BwdArgs& a, int b, int g, int kt, F32KvSmem<DQK, DV>& sm) {
  using C = F32BCfg<DQK, DV>;
  constexpr int BQ = C::BQK, BKEY = C::BKEY, QS = C::QS, OS = C::OS, KS = C::KS, VS = C::VS, PS2 = C::PS2;
  constexpr int T = C::THREADS;   // threads per half
  constexpr int KK = C::KK, KVV = C::KVV;
  static_assert(T * (KK + KVV) * 16 <= BKEY * (KS + VS) * 4, "partial sums fit the K / V area");
  const int tid = threadIdx.x, half = tid / T, lt = tid % T;
  const int key_base = kt * BKEY;
  int q_first = 0;   // the first query that can see the tile's first key
  if (a.causal) {
    const long long f = a.k_pos0 + key_base - a.q_pos0;
    q_first = (int)max(0LL, min(f, (long long)a.Sq));
  }
  if (q_first >= a.Sq) return;   // no query of the block sees these keys
  const int qt0 = q_first / BQ;
  const int nqt = (a.Sq + BQ - 1) / BQ - qt0;
  const int ntiles = a.group * nqt;   // (query head of the group, query tile) pairs
  const int niter = (ntiles + 1) / 2; // half h takes pairs 2 i + h

  float* ksm = sm.kv;
  float* vsm = sm.kv + BKEY * KS;
  float* qsm = sm.q[half];
  float* osm = sm.o[half];
  float* psm = sm.p[half];
  float* dssm = sm.ds[half];
  const size_t kvh = (size_t)(b * a.Hkv + g) * a.Sk;
  __syncthreads();   // the previous tile's K, V and partial sums are consumed
  for (int e = tid; e < BKEY * DQK / 4; e += 2 * T) {
    const int rr = e / (DQK / 4), c4 = e % (DQK / 4), key = key_base + rr;
    *(float4*)&ksm[rr * KS + 4 * c4] = key < a.Sk ? *(const float4*)((const float*)a.k + (kvh + key) * DQK + 4 * c4)
                                                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int e = tid; e < BKEY * DV / 4; e += 2 * T) {
    const int rr = e / (DV / 4), c4 = e % (DV / 4), key = key_base + rr;
    *(float4*)&vsm[rr * VS + 4 * c4] = key < a.Sk ? *(const float4*)((const float*)a.v + (kvh + key) * DV + 4 * c4)
                                                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // phase 1 (P, dS): keys kp, kp + 16 against rows rq, rq + 16, kp = t % 16,
  // rq = t / 16. Phase 2: dK columns 4 (t % (DQK/4)) .. + 3 of keys KK (t / (DQK/4))
  // .. + KK - 1, and dV likewise (t: the thread's index in its half).
  const int kp = lt & 15, rq = lt >> 4;
  const int cgk = lt % (DQK / 4), kgk = lt / (DQK / 4);
  const int cgv = lt % (DV / 4), kgv = lt / (DV / 4);
  const long long kpos_a = a.k_pos0 + key_base + kp;
  const bool key_a_ok = key_base + kp < a.Sk, key_b_ok = key_base + kp + 16 < a.Sk;
  float4 acck[KK], accv[KVV];
#pragma unroll
  for (int m = 0; m < KK; ++m) acck[m] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < KVV; ++m) accv[m] = make_float4(0.f, 0.f, 0.f, 0.f);

  // the half's next (head, query tile): rows and statistics fetched one step ahead
  float4 qr[C::QCH2], orr[C::OCH2];
  float l2n = kNegInf, dln = 0.f;
  auto fetch = [&](int n) {
    const int hq = g * a.group + n / nqt, row0 = (qt0 + n % nqt) * BQ;
    const size_t bh = (size_t)b * a.Hq + hq;
    load_rows<DQK, C::QCH2, T>(qr, (const float*)a.q + bh * a.Sq * DQK, row0, a.Sq, lt);
    load_rows<DV, C::OCH2, T>(orr, (const float*)a.dout + bh * a.Sq * DV, row0, a.Sq, lt);
    if (lt < BQ) {
      // -LSE * log2(e) of each row (-inf past the block or with no visible key: P = 0)
      const int row = row0 + lt;
      l2n = kNegInf;
      dln = 0.f;
      if (row < a.Sq) {
        const float l = a.lse[bh * a.Sq + row];
        if (l != kNegInf) l2n = -l * kLog2e;
        dln = a.delta[bh * a.Sq + row];
      }
    }
  };
  if (half < ntiles) fetch(half);
  for (int it = 0; it < niter; ++it) {
    const int n = 2 * it + half;
    const bool active = n < ntiles;   // the second half idles on an odd count's last step
    const int row0 = (qt0 + n % nqt) * BQ;
    __syncthreads();   // the previous pair's rows, P and dS are consumed
    if (active) {
      store_rows<DQK, C::QCH2, T, QS>(qr, qsm, lt);
      store_rows<DV, C::OCH2, T, OS>(orr, osm, lt);
      if (lt < BQ) {
        sm.l2[half][lt] = l2n;
        sm.dl[half][lt] = dln;
      }
    }
    __syncthreads();   // the pair's rows and statistics (and the K, V rows) are in LDS
    if (n + 2 < ntiles) fetch(n + 2);   // lands while this pair is computed
    if (active) {
      float s00 = 0.f, s01 = 0.f, s10 = 0.f, s11 = 0.f;   // s[row][key]
#pragma unroll 4
      for (int d4 = 0; d4 < DQK / 4; ++d4) {
        const float4 k0 = lds4(&ksm[kp * KS + 4 * d4]), k1 = lds4(&ksm[(kp + 16) * KS + 4 * d4]);
        const float4 q0 = lds4(&qsm[rq * QS + 4 * d4]), q1 = lds4(&qsm[(rq + 16) * QS + 4 * d4]);
        s00 = dot4(q0, k0, s00);
        s01 = dot4(q0, k1, s01);
        s10 = dot4(q1, k0, s10);
        s11 = dot4(q1, k1, s11);
      }
      float p00 = 0.f, p01 = 0.f, p10 = 0.f, p11 = 0.f;   // dP[row][key]
#pragma unroll 4
      for (int d4 = 0; d4 < DV / 4; ++d4) {
        const float4 v0 = lds4(&vsm[kp * VS + 4 * d4]), v1 = lds4(&vsm[(kp + 16) * VS + 4 * d4]);
        const float4 o0 = lds4(&osm[rq * OS + 4 * d4]), o1 = lds4(&osm[(rq + 16) * OS + 4 * d4]);
        p00 = dot4(o0, v0, p00);
        p01 = dot4(o0, v1, p01);
        p10 = dot4(o1, v0, p10);
        p11 = dot4(o1, v1, p11);
      }
      const long long qpos = a.q_pos0 + row0 + rq;
      const float l0 = sm.l2[half][rq], l1 = sm.l2[half][rq + 16];
      const float dl0 = sm.dl[half][rq], dl1 = sm.dl[half][rq + 16];
      auto prob = [&](float sv, bool ok, long long kpos, long long qp, float l) {
        return ok && (!a.causal || kpos <= qp) ? exp2_hw(fmaf(sv, a.scale_log2, l)) : 0.f;
      };
      const float pa0 = prob(s00, key_a_ok, kpos_a, qpos, l0), pb0 = prob(s01, key_b_ok, kpos_a + 16, qpos, l0);
      const float pa1 = prob(s10, key_a_ok, kpos_a, qpos + 16, l1);
      const float pb1 = prob(s11, key_b_ok, kpos_a + 16, qpos + 16, l1);
      psm[rq * PS2 + kp] = pa0;
      psm[rq * PS2 + kp + 16] = pb0;
      psm[(rq + 16) * PS2 + kp] = pa1;
      psm[(rq + 16) * PS2 + kp + 16] = pb1;
      dssm[rq * PS2 + kp] = pa0 * (p00 - dl0);
      dssm[rq * PS2 + kp + 16] = pb0 * (p01 - dl0);
      dssm[(rq + 16) * PS2 + kp] = pa1 * (p10 - dl1);
      dssm[(rq + 16) * PS2 + kp + 16] = pb1 * (p11 - dl1);
    }
    __syncthreads();   // P and dS of the pair are in LDS
    if (active) {
#pragma unroll 2
      for (int rr = 0; rr < BQ; ++rr) {
        float ds[KK], p[KVV];
        lds_n<KK>(ds, &dssm[rr * PS2 + KK * kgk]);
        lds_n<KVV>(p, &psm[rr * PS2 + KVV * kgv]);
        const float4 qx = lds4(&qsm[rr * QS + 4 * cgk]);
        const float4 ox = lds4(&osm[rr * OS + 4 * cgv]);
#pragma unroll
        for (int m = 0; m < KK; ++m) axpy4(ds[m], qx, acck[m]);
#pragma unroll
        for (int m = 0; m < KVV; ++m) axpy4(p[m], ox, accv[m]);
      }
    }
  }

  // the second half's sums join the first half's through the K / V area
  float4* red = (float4*)sm.kv;
  __syncthreads();   // every read of K and V is done
  if (half == 1) {
#pragma unroll
    for (int m = 0; m < KK; ++m) red[m * T + lt] = acck[m];
#pragma unroll
    for (int m = 0; m < KVV; ++m) red[(KK + m) * T + lt] = accv[m];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int m = 0; m < KK; ++m) {
      const int key = key_base + KK * kgk + m;
      if (key < a.Sk) {
        const float4 o2 = red[m * T + lt];
        float4 sum = acck[m];
        sum.x += o2.x;
        sum.y += o2.y;
        sum.z += o2.z;
        sum.w += o2.w;
        float* dkp = a.dk + (kvh + key) * DQK + 4 * cgk;
        float4 cur = *(const float4*)dkp;
        axpy4(a.scale, sum, cur);
        *(float4*)dkp = cur;
      }
    }
#pragma unroll
    for (int m = 0; m < KVV; ++m) {
      const int key = key_base + KVV * kgv + m;
      if (key < a.Sk) {
        const float4 o2 = red[(KK + m) * T + lt];
        float* dvp = a.dv + (kvh + key) * DV + 4 * cgv;
        float4 cur = *(const float4*)dvp;
        cur.x += accv[m].x + o2.x;
        cur.y += accv[m].y + o2.y;
        cur.z += accv[m].z + o2.z;
        cur.w += accv[m].w + o2.w;
        *(float4*)dvp = cur;
      }
    }
  }
}

// Under a causal mask a workgroup takes key tiles kt and n - 1 - kt of one (batch,
// KV head), one after the other: the first sees about as many query tiles as the
// second misses, so every workgroup has about the same work; with fewer workgroups
// than the chip holds at once, an unpaired grid would last as long as its first
// (heaviest) tile. Without a mask every tile has the same work and a workgroup
// takes one.
template <int DQK, int DV>
// Two waves per SIMD: one workgroup per CU, with the registers to keep more LDS
// reads in flight (at D = 128 the compiler otherwise holds the kernel to the 128
// registers of two workgroups per CU and serialises the reads).
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_f32_kernel(BwdArgs a) {
  using C = F32BCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) F32KvSmem<DQK, DV> sm;
  const int nkt = (a.Sk + C::BKEY - 1) / C::BKEY;
  const int kt = (int)(blockIdx.x % a.n_tiles);   // a.n_tiles: ceil(nkt / 2) causal, nkt otherwise
  const int bg = blockIdx.x / a.n_tiles;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  dkdv_f32_tile<DQK, DV>(a, b, g, kt, sm);
  if (a.causal && nkt - 1 - kt != kt) dkdv_f32_tile<DQK, DV>(a, b, g, nkt - 1 - kt, sm);
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
  using C = F32BCfg<DQK, DV>;
  BwdArgs b = a;
  const int nkt = (a.Sk + C::BKEY - 1) / C::BKEY;
  b.n_tiles = a.causal ? (nkt + 1) / 2 : nkt;   // causal: pairs of key tiles
  long long grid = (long long)a.B * a.Hkv * b.n_tiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid > 0)
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<DQK, DV>), dim3((unsigned)grid), dim3(2 * C::THREADS), 0, st, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 32-row dQ workgroups (two rows per thread), or 16-row ones when there are fewer
  // 32-row workgroups than CUs
  const bool two_rows = (long long)a.B * a.Hq * ((a.Sq + 31) / 32) >= 256;
  b.n_tiles = two_rows ? (a.Sq + 31) / 32 : (a.Sq + 15) / 16;
  grid = (long long)a.B * a.Hq * b.n_tiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid > 0) {
    if (two_rows)
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DQK, DV, 2>), dim3((unsigned)grid), dim3(C::THREADS), 0, st, b);
    else
      hipLaunchKernelGGL((bwd_dq_f32_kernel<DQK, DV, 1>), dim3((unsigned)grid), dim3(C::THREADS), 0, st, b);
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
