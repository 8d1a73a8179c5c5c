// Backward pass of blockwise exact attention for gfx950 (bf16 inputs, fp32
// gradient accumulators), on v_mfma_f32_32x32x16_bf16.
//
// What is computed: the exact gradients of O = softmax(scale * Q K^T) V over the
// visible keys, for one (query block, KV block) pair at a time, given the
// queries' full-row LSE saved by the forward pass and delta = rowsum(dO o O)
// (page "长上下文的第一性挑战", §挑战 1, eq. lc-ch-attention is the function
// differentiated; page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算
// 一条超长序列", §什么时候值得引入 Context Parallelism, names the backward pass's
// data dependencies among what a ring must get right). With P = exp(scale q k -
// LSE) restricted to the block, each pair adds
//     dV += P^T dO,  dS = P o (dO V^T - delta),  dQ += scale dS K,  dK += scale dS^T Q
// to fp32 accumulators, so a ring backward is P such steps per device with dK / dV
// travelling with their KV block; the sums are order independent.
//
// Three kernels:
//   * bwd_delta_kernel: delta = rowsum(dO o O) per query row.
//   * Scores are fp32 products of the bf16 inputs; P = exp2(scale * log2(e) * s
//     - LSE * log2(e)). The dP products start from -delta (their C operand), so they
//     come out as dP - delta. In the dK/dV kernel the S products likewise start from
//     -LSE / scale, so P = exp2(scale * log2(e) * (S - LSE / scale)).
//   * bwd_dq_kernel: one workgroup per 256 query rows of one (batch, head), 8 waves
//     of 32 rows. Q and dO rows stay in VGPRs as B operands (lane = query column;
//     at D_qk = 192 the dO rows wait in a lane-private LDS area instead); K and V
//     tiles are staged in LDS (double buffered). Per 32 keys: S^T = K Q^T and
//     dP^T = V dO^T (lane-local LSE and delta), dS^T, then dQ^T += K^T dS^T with
//     K^T read through ds_read_b64_tr_b16. K / V tiles are 128 keys (64 at D_qk = 192).
//   * bwd_dkdv_kernel: one workgroup per 256 keys of one (batch, KV head), 8 waves
//     of 32 keys, looping over the group's query heads and the visible query tiles
//     (64 rows, 32 at D_qk = 192, loaded straight from HBM into LDS, with their LSE
//     and delta). K and V rows stay in VGPRs as the B operands of S = Q K^T and
//     dP = dO V^T (lane = key column; at D_qk = 192 the K rows wait in a
//     lane-private LDS area instead). dV^T += dO^T P and dK^T += Q^T dS take dO^T
//     and Q^T through ds_read_b64_tr_b16. Rows past the query block carry
//     LSE = +inf (their S products start from -inf), so their P and dS are
//     exactly 0 with no row mask.
#include "common.hpp"

namespace ra {

constexpr float kPosInf = __builtin_huge_valf();

// ---- delta = rowsum(dO o O) ----------------------------------------------------------
// A 16-lane group per row: Dv/8 16-byte chunks over the group, then a butterfly sum.
__global__ void __launch_bounds__(256)
bwd_delta_kernel(const __bf16* o, const __bf16* dout, float* delta, long long rows, int Dv) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int L = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    for (int c = L; c < Dv / 8; c += 16) {
      const bf16x8 x = *(const bf16x8*)(o + row * Dv + c * 8);
      const bf16x8 y = *(const bf16x8*)(dout + row * Dv + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (row < rows && L == 0) delta[row] = acc;
}

// LDS row strides (elements): every tile row is padded by 8 elements, so 16
// consecutive rows start on 16 different 4-bank groups (16-byte row reads are free
// of bank conflicts). K (dQ kernel), Q and dO (dK/dV kernel) are also read
// transposed; for those the row order below keeps the transposed reads conflict-free.
// (D + 8)-element rows start 4 (D = 64, 128) or 36 (D = 192) banks apart, which
// serves both reads below alike.
//
// NW = 8 waves of 32 rows (dQ) or keys (dK, dV) per workgroup, two per SIMD. At
// D_qk = 192, D_v = 128 a wave's working set does not fit the 256 registers of
// two waves per SIMD as it does at D = 128: the dK/dV kernel's dK^T and dV^T
// accumulators of 32 keys take 160 registers beside 80 of K and V rows, the dQ
// kernel's dQ^T 96 beside 80 of Q and dO rows. There one stationary operand moves
// to a lane-private LDS area: each lane stores its own 16-byte chunks once and
// reads back only those, so no barrier is involved. The dK/dV kernel parks its K
// rows (96 KB beside 32-row Q and dO tiles: 141 KB) and runs at 254 VGPRs; the dQ
// kernel parks its dO rows (64 KB beside 64-key K and V tiles: 148 KB), 239 VGPRs.
template <int DQK, int DV, int NW>
struct BCfg {
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = NW * 32;              // query rows (dQ) / keys (dK, dV) per workgroup
  static constexpr int BK = DQK > 128 ? 64 : 128;   // keys per LDS tile (dQ kernel): two K + V tiles fit
  static constexpr int BQ = DQK > 128 ? 32 : 64;    // query rows per LDS tile (dK/dV kernel; 32 leaves room for the K rows)
  static constexpr int KS = DQK + 8, VS = DV + 8, OS = DV + 8;
  static constexpr int DS = DQK / 16, DSV = DV / 16;  // MFMA k-steps
  static constexpr int MT = DQK / 32, MTV = DV / 32;  // 32-row output tiles
};
// Waves per workgroup of both kernels.
constexpr int kBwdWaves = 8;
// D_qk = 192: the K rows (dK/dV kernel) and the dO rows (dQ kernel) of each wave sit
// in a lane-private LDS area instead of VGPRs (each lane reads back only the 16-byte
// chunks it wrote, so no barrier is needed)
template <int DQK, int DV>
constexpr bool dkdv_k_in_lds() { return DQK > 128; }
template <int DQK, int DV>
constexpr bool dq_o_in_lds() { return DQK > 128; }

// Row order inside each 16-row block of a tile read both as rows and transposed: the
// MFMA row (accumulator row) 4a + b reads LDS row 4b + a (an involution). A half
// wave's transposed read takes 64 bytes from each of 4 consecutive accumulator rows
// 4a .. 4a+3; they sit in LDS rows a, a+4, a+8, a+12, which with (D + 8)-element rows
// start 16 banks apart, so the 4 x 64 bytes cover all 64 banks once. The 16-byte row
// reads of 16 consecutive accumulator rows still touch 16 distinct LDS rows.
__device__ __forceinline__ int perm16(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// ---- dQ -------------------------------------------------------------------------------
template <int DQK, int DV, int NW>
__global__ void __launch_bounds__(NW * 64)
bwd_dq_kernel(BwdArgs a) {
  using C = BCfg<DQK, DV, NW>;
  constexpr int BK = C::BK;
  constexpr int KCH = BK * DQK / 8 / C::THREADS, VCH = BK * DV / 8 / C::THREADS;
  static_assert(KCH * C::THREADS * 8 == BK * DQK && VCH * C::THREADS * 8 == BK * DV, "tile split");
  constexpr bool OLDS = dq_o_in_lds<DQK, DV>();
  // the direct loads fill whole 1 KB pieces, so each tile is allocated in whole KB
  __shared__ __attribute__((aligned(16))) __bf16 ks[2][padded_tile_bytes(BK, C::KS * 2) / 2];
  __shared__ __attribute__((aligned(16))) __bf16 vs[2][padded_tile_bytes(BK, C::VS * 2) / 2];
  // lane-private dO rows (OLDS): lane (wave, l32, h) holds chunk 16 s + 8 h of row l32
  __shared__ __attribute__((aligned(16))) bf16x8 osm[OLDS ? NW * C::DSV * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5, gg = lane >> 4, L = lane & 15;
  // XCD-aware order (as the forward): XCD x runs the x-th eighth of the work list
  // (batch, KV head, query tile from the last, query head of the group), so the
  // co-resident workgroups of an XCD stream the same K/V tiles through its L2.
  const int n_items = a.B * a.Hq * a.n_tiles;
  const int per_xcd = (n_items + 7) >> 3;
  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= n_items) return;
  const int w = u % a.group, rest = u / a.group;
  const int qt = a.n_tiles - 1 - rest % a.n_tiles;
  const int bgi = rest / a.n_tiles;
  const int b = bgi / a.Hkv, g = bgi - b * a.Hkv, hq = g * a.group + w;
  const int bh = b * a.Hq + hq;
  const int row_base = qt * C::ROWS;
  const int last_row = min(row_base + C::ROWS, a.Sq) - 1;
  long long kmax = a.Sk;
  if (a.causal) kmax = min(kmax, a.q_pos0 + last_row - a.k_pos0 + 1);
  if (kmax <= 0) return;  // no key of the block is visible to this tile
  const int ntiles = (int)((kmax + BK - 1) / BK);

  const size_t kvh = (size_t)(b * a.Hkv + g) * a.Sk;
  const auto qrs = make_rsrc((const __bf16*)a.q + (size_t)bh * a.Sq * DQK, (unsigned)((size_t)a.Sq * DQK * 2));
  const auto ors = make_rsrc((const __bf16*)a.dout + (size_t)bh * a.Sq * DV, (unsigned)((size_t)a.Sq * DV * 2));
  const auto krs = make_rsrc((const __bf16*)a.k + kvh * DQK, (unsigned)((size_t)a.Sk * DQK * 2));
  const auto vrs = make_rsrc((const __bf16*)a.v + kvh * DV, (unsigned)((size_t)a.Sk * DV * 2));

  const int wave_row0 = row_base + wave * 32;
  const long long wave_pos0 = a.q_pos0 + wave_row0;
  const int my_row = wave_row0 + l32;
  bf16x8 qf[C::DS], of[OLDS ? 1 : C::DSV];
#pragma unroll
  for (int s = 0; s < C::DS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (unsigned)(my_row * DQK + 16 * s + 8 * h) * 2u));
  // conflict-free: consecutive lanes take consecutive 16-byte slots
  auto oslot = [&](int s) -> bf16x8& { return osm[(wave * C::DSV + s) * 64 + lane]; };
  if constexpr (OLDS) {
#pragma unroll
    for (int s = 0; s < C::DSV; ++s)
      oslot(s) = __builtin_bit_cast(bf16x8, buf_load16(ors, (unsigned)(my_row * DV + 16 * s + 8 * h) * 2u));
  } else {
#pragma unroll
    for (int s = 0; s < C::DSV; ++s)
      of[s] = __builtin_bit_cast(bf16x8, buf_load16(ors, (unsigned)(my_row * DV + 16 * s + 8 * h) * 2u));
  }
  // a row past the block, or with no visible key at all, gets P = 0
  float lse2 = kPosInf, dlt = 0.f;
  if (my_row < a.Sq) {
    const float l = a.lse[(size_t)bh * a.Sq + my_row];
    if (l != kNegInf) lse2 = l * kLog2e;
    dlt = a.delta[(size_t)bh * a.Sq + my_row];
  }
  constexpr bool DMA = (DQK == 128 && DV == 128) || DQK == 192;
  f32x16 dqacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) dqacc[mt] = f32x16{};

  // D = 128: tiles go straight from HBM into the padded LDS rows
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  PaddedTileDma<BK, DQK * 2, C::KS * 2, NW> kdma;
  PaddedTileDma<BK, DV * 2, C::VS * 2, NW> vdma;
  static_assert(sizeof(ks[0]) == decltype(kdma)::PIECES * 1024 && sizeof(vs[0]) == decltype(vdma)::PIECES * 1024,
                "every 1 KB piece of a tile's direct loads lands inside that tile");
  if constexpr (DMA) {
    kdma.init(wave_u, lane);
    vdma.init(wave_u, lane);
  }
  const u32x4 kdesc = raw_desc((const __bf16*)a.k + kvh * DQK, (unsigned)((size_t)a.Sk * DQK * 2));
  const u32x4 vdesc = raw_desc((const __bf16*)a.v + kvh * DV, (unsigned)((size_t)a.Sk * DV * 2));
  auto dma_tile = [&](int n, int buf) {
    kdma.issue(wave_u, lds_addr(&ks[buf][0]), (unsigned)(n * BK * DQK * 2), (unsigned)(a.Sk * DQK * 2 - 16), kdesc);
    vdma.issue(wave_u, lds_addr(&vs[buf][0]), (unsigned)(n * BK * DV * 2), (unsigned)(a.Sk * DV * 2 - 16), vdesc);
  };
  uint4 kr[DMA ? 1 : KCH], vr[DMA ? 1 : VCH];
  auto load_tile = [&](int n) {
    const int row0 = n * BK;
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int c = it * C::THREADS + tid, row = c / (DQK / 8), col = c % (DQK / 8);
      kr[it] = buf_load16(krs, (unsigned)((row0 + row) * DQK + col * 8) * 2u);
    }
#pragma unroll
    for (int it = 0; it < VCH; ++it) {
      const int c = it * C::THREADS + tid, row = c / (DV / 8), col = c % (DV / 8);
      vr[it] = buf_load16(vrs, (unsigned)((row0 + row) * DV + col * 8) * 2u);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int c = it * C::THREADS + tid, row = c / (DQK / 8), col = c % (DQK / 8);
      *(uint4*)&ks[buf][row * C::KS + col * 8] = kr[it];
    }
#pragma unroll
    for (int it = 0; it < VCH; ++it) {
      const int c = it * C::THREADS + tid, row = c / (DV / 8), col = c % (DV / 8);
      *(uint4*)&vs[buf][row * C::VS + col * 8] = vr[it];
    }
  };

  auto compute_tile = [&](int buf, long long kpos0, int nvalid, bool need_mask) {
#pragma unroll
    for (int kt = 0; kt < BK / 32; ++kt) {
      const int krow = kt * 32 + perm16(l32);   // the key of accumulator row l32
      // dP^T starts from -delta, so it comes out as dP - delta
      f32x16 st = f32x16{}, dpt;
#pragma unroll
      for (int i = 0; i < 16; ++i) dpt[i] = -dlt;
      // S^T and dP^T as two chains (DS and DSV steps; the longer one runs on
      // alone), each step's K and V fragments read while the previous step's
      // products run
      constexpr int NSTEP = C::DS > C::DSV ? C::DS : C::DSV;
      bf16x8 kc = *(const bf16x8*)&ks[buf][krow * C::KS + 8 * h];
      bf16x8 vc = *(const bf16x8*)&vs[buf][krow * C::VS + 8 * h];
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        bf16x8 kn = kc, vn = vc;
        if (s + 1 < C::DS) kn = *(const bf16x8*)&ks[buf][krow * C::KS + 16 * (s + 1) + 8 * h];
        if (s + 1 < C::DSV) vn = *(const bf16x8*)&vs[buf][krow * C::VS + 16 * (s + 1) + 8 * h];
        __builtin_amdgcn_sched_barrier(0);
        if (s < C::DS) st = mfma32(kc, qf[s], st);
        if (s < C::DSV) {
          if constexpr (OLDS)
            dpt = mfma32(vc, oslot(s), dpt);
          else
            dpt = mfma32(vc, of[s], dpt);
        }
        __builtin_amdgcn_sched_barrier(0);
        kc = kn;
        vc = vn;
      }
      if (need_mask) {
        // last visible key of this 32-key block for the lane's query, minus h;
        // element i holds accumulator row 8*(i/4) + 4*h + i%4, i.e. the key at
        // perm16 of it: 16*(i/8) + 4*(i%4) + 2*((i/4)%2) + h
        int lim = nvalid - 1 - kt * 32;
        if (a.causal) {
          const long long rel = wave_pos0 + l32 - (kpos0 + kt * 32);
          lim = (int)min((long long)lim, max(rel, -1LL));
        }
        lim -= h;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) > lim) st[i] = kNegInf;
      }
      // dS^T = P^T o (dP^T - delta), rounded to bf16 as the B operand of dQ^T
      bf16x8 dsb[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * t2 + e;
          x[e] = exp2_hw(fmaf(st[i], a.scale_log2, -lse2)) * dpt[i];
        }
        dsb[t2] = to_bf16x8(x);
      }
      // dQ^T += K^T dS^T: step t2 holds accumulator rows 16*t2 + 4*h + {0..3} and
      // 16*t2 + 8 + 4*h + {0..3} in lane half h; K^T rows d = 32*mt + lane%32. The
      // transposed read of accumulator row 16*t2 + 8*x + 4*(gg/2) + L/4 takes its
      // key's LDS row, perm16 of it.
      auto ktread = [&](int mt, bf16x4 (&f)[2][2]) {
        const int dcol = 32 * mt + 16 * (gg & 1) + 4 * (L & 3);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int key = kt * 32 + 16 * t2 + 4 * (L >> 2) + 2 * x + (gg >> 1);
            f[t2][x] = lds_read_tr16(&ks[buf][key * C::KS + dcol]);
          }
      };
      // K^T fragments of output tile mt + 1 read while the products of mt run
      bf16x4 fc[2][2], fn[2][2];
      ktread(0, fc);
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        if (mt + 1 < C::MT) ktread(mt + 1, fn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) dqacc[mt] = mfma32(cat(fc[t2][0], fc[t2][1]), dsb[t2], dqacc[mt]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int x = 0; x < 2; ++x) fc[t2][x] = fn[t2][x];
      }
    }
  };

  if constexpr (DMA) {
    dma_tile(0, 0);
    wait_vmem();
  } else {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  if (!DMA && ntiles > 1) load_tile(1);
  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    const long long kpos0 = a.k_pos0 + (long long)n * BK;
    const int nvalid = min(BK, a.Sk - n * BK);
    // the other buffer was last read before the previous barrier
    if (DMA && n + 1 < ntiles) dma_tile(n + 1, buf ^ 1);
    const bool skip = a.causal && kpos0 > wave_pos0 + 31;
    const bool need_mask = nvalid < BK || (a.causal && kpos0 + BK - 1 > wave_pos0);
    if (!skip) compute_tile(buf, kpos0, nvalid, need_mask);
    if (DMA) {
      wait_vmem();   // this wave's loads of tile n+1 have landed
    } else if (n + 1 < ntiles) {
      store_tile(buf ^ 1);
      if (n + 2 < ntiles) load_tile(n + 2);
    }
    __syncthreads();
  }

  if (my_row < a.Sq) {
    float* dqp = a.dq + ((size_t)bh * a.Sq + my_row) * DQK;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * mt + 8 * g4 + 4 * h;
        f32x4 cur = *(const f32x4*)(dqp + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[e] = fmaf(a.scale, dqacc[mt][4 * g4 + e], cur[e]);
        *(f32x4*)(dqp + d) = cur;
      }
  }
}

// ---- dK, dV ---------------------------------------------------------------------------
template <int DQK, int DV, int NW>
__global__ void __launch_bounds__(NW * 64)
bwd_dkdv_kernel(BwdArgs a) {
  using C = BCfg<DQK, DV, NW>;
  constexpr int BQ = C::BQ;
  constexpr int QS = C::KS, OS = C::OS;   // Q rows like K rows
  // the direct loads fill whole 1 KB pieces, so each tile is allocated in whole KB
  // (32 rows of 400 or 272 bytes are not)
  __shared__ __attribute__((aligned(16))) __bf16 qsm[2][padded_tile_bytes(BQ, QS * 2) / 2];
  __shared__ __attribute__((aligned(16))) __bf16 osm[2][padded_tile_bytes(BQ, OS * 2) / 2];
  __shared__ __attribute__((aligned(16))) float lsm[2][BQ];
  __shared__ __attribute__((aligned(16))) float dsm[2][BQ];
  constexpr bool KLDS = dkdv_k_in_lds<DQK, DV>();
  // lane-private K row chunks (KLDS): lane (wave, l32, h) holds chunk 16 s + 8 h of its key
  __shared__ __attribute__((aligned(16))) bf16x8 kpriv[KLDS ? NW * C::DS * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: derived positions stay scalar
  const int l32 = lane & 31, h = lane >> 5, gg = lane >> 4, L = lane & 15;
  // XCD-aware order: XCD x runs the x-th eighth of the work list (batch, KV head,
  // key tile), so its co-resident workgroups stream the same Q / dO tiles through
  // its L2; under a causal mask the first key tiles (the most queries) go first.
  const int n_items = a.B * a.Hkv * a.n_tiles;
  const int per_xcd = (n_items + 7) >> 3;
  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= n_items) return;
  const int ktile = u % a.n_tiles;
  const int bg = u / a.n_tiles;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int key_base = ktile * C::ROWS;

  // queries that can see the workgroup's first key (all of them without a mask)
  int q_first = 0;
  if (a.causal) {
    const long long f = a.k_pos0 + key_base - a.q_pos0;
    q_first = (int)max(0LL, min(f, (long long)a.Sq));
  }
  if (q_first >= a.Sq) return;  // no query of the block sees these keys
  const int qt0 = q_first / BQ;
  const int nqt = (a.Sq + BQ - 1) / BQ - qt0;
  const int ntiles = a.group * nqt;   // (query head of the group, query tile) pairs

  const size_t kvh = (size_t)bg * a.Sk;
  const auto krs = make_rsrc((const __bf16*)a.k + kvh * DQK, (unsigned)((size_t)a.Sk * DQK * 2));
  const auto vrs = make_rsrc((const __bf16*)a.v + kvh * DV, (unsigned)((size_t)a.Sk * DV * 2));
  const int wave_key0 = key_base + wave * 32;
  const long long wave_kpos0 = a.k_pos0 + wave_key0;
  const int my_key = wave_key0 + l32;

  // K row of the lane's key as the B operand of S = Q K^T (keys past the block read 0)
  bf16x8 kf[KLDS ? 1 : C::DS];
  auto kslot = [&](int s) -> bf16x8& { return kpriv[(wave * C::DS + s) * 64 + lane]; };
#pragma unroll
  for (int s = 0; s < C::DS; ++s) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, buf_load16(krs, (unsigned)(my_key * DQK + 16 * s + 8 * h) * 2u));
    if constexpr (KLDS)
      kslot(s) = x;
    else
      kf[s] = x;
  }
  // V row of the lane's key as the B operand of dP = dO V^T
  bf16x8 vf[C::DSV];
#pragma unroll
  for (int s = 0; s < C::DSV; ++s)
    vf[s] = __builtin_bit_cast(bf16x8, buf_load16(vrs, (unsigned)(my_key * DV + 16 * s + 8 * h) * 2u));
  f32x16 dkacc[C::MT], dvacc[C::MTV];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) dkacc[mt] = f32x16{};
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) dvacc[mt] = f32x16{};

  // Q / dO tiles go straight from HBM into the padded LDS rows (rows past the block
  // re-read the slab's last 16 bytes: finite values whose P is 0); the rows' LSE and
  // delta go through a register of threads 0..127
  float rowv = 0.f;   // threads 0..BQ-1: -LSE / scale of a row; BQ..2BQ-1: -delta
  static_assert(C::THREADS >= 2 * BQ, "threads 0 .. 2 BQ - 1 carry the rows' LSE and delta");
  PaddedTileDma<BQ, DQK * 2, QS * 2, NW> qdma;
  PaddedTileDma<BQ, DV * 2, OS * 2, NW> odma;
  static_assert(sizeof(qsm[0]) == decltype(qdma)::PIECES * 1024 && sizeof(osm[0]) == decltype(odma)::PIECES * 1024,
                "every 1 KB piece of a tile's direct loads lands inside that tile");
  qdma.init(wave, lane);
  odma.init(wave, lane);
  auto tile_head = [&](int n) { return g * a.group + n / nqt; };
  auto tile_row0 = [&](int n) { return (qt0 + n % nqt) * BQ; };
  auto load_tile = [&](int n, int buf) {
    const int hq = tile_head(n), row0 = tile_row0(n);
    const size_t bh = (size_t)b * a.Hq + hq;
    if (tid < 2 * BQ) {
      const int r = row0 + (tid & (BQ - 1));
      if (tid < BQ) {
        rowv = kNegInf;   // rows past the block, or with no visible key: P = 0
        if (r < a.Sq) {
          const float l = a.lse[bh * a.Sq + r];
          if (l != kNegInf) rowv = -l / a.scale;
        }
      } else {
        rowv = r < a.Sq ? -a.delta[bh * a.Sq + r] : 0.f;
      }
    }
    const u32x4 qdesc = raw_desc((const __bf16*)a.q + bh * a.Sq * DQK, (unsigned)((size_t)a.Sq * DQK * 2));
    const u32x4 odesc = raw_desc((const __bf16*)a.dout + bh * a.Sq * DV, (unsigned)((size_t)a.Sq * DV * 2));
    qdma.issue(wave, lds_addr(&qsm[buf][0]), (unsigned)(row0 * DQK * 2), (unsigned)(a.Sq * DQK * 2 - 16), qdesc);
    odma.issue(wave, lds_addr(&osm[buf][0]), (unsigned)(row0 * DV * 2), (unsigned)(a.Sq * DV * 2 - 16), odesc);
  };
  auto store_rows = [&](int buf) {
    // LSE and delta are kept in accumulator-row order (perm16 is its own inverse)
    if (tid < BQ)
      lsm[buf][perm16(tid)] = rowv;
    else if (tid < 2 * BQ)
      dsm[buf][perm16(tid - BQ)] = rowv;
  };

  auto compute_tile = [&](int buf, long long qpos_t) {
#pragma unroll
    for (int qs = 0; qs < BQ / 32; ++qs) {
      const long long qpos_s = qpos_t + qs * 32;
      if (a.causal && qpos_s + 31 < wave_kpos0) continue;   // these queries precede all the wave's keys
      const bool need_mask = a.causal && qpos_s < wave_kpos0 + 31;
      const int qrow = qs * 32 + perm16(l32);   // the query of accumulator row l32
      // S = Q K^T and dP = dO V^T: lane = key column, accumulator rows 8*(i/4) + 4*h +
      // i%4 (their queries at perm16 of that). S starts from the rows' -LSE / scale
      // and dP from their -delta, so they come out as S - LSE / scale and dP - delta:
      // P = exp2(scale * log2(e) * (S - LSE / scale)) needs one multiply per score,
      // and the rows' LSE is read before the products instead of between them and
      // the exps. The offset costs the fp32 accumulation a few ulps of |S - LSE /
      // scale|, far below the bf16 rounding of P.
      f32x16 st, dpt;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const f32x4 l0 = *(const f32x4*)&lsm[buf][qs * 32 + 16 * t2 + 4 * h];
        const f32x4 l1 = *(const f32x4*)&lsm[buf][qs * 32 + 16 * t2 + 8 + 4 * h];
        const f32x4 d0 = *(const f32x4*)&dsm[buf][qs * 32 + 16 * t2 + 4 * h];
        const f32x4 d1 = *(const f32x4*)&dsm[buf][qs * 32 + 16 * t2 + 8 + 4 * h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st[8 * t2 + e] = l0[e];
          st[8 * t2 + 4 + e] = l1[e];
          dpt[8 * t2 + e] = d0[e];
          dpt[8 * t2 + 4 + e] = d1[e];
        }
      }
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        if constexpr (KLDS)
          st = mfma32(*(const bf16x8*)&qsm[buf][qrow * QS + 16 * s + 8 * h], kslot(s), st);
        else
          st = mfma32(*(const bf16x8*)&qsm[buf][qrow * QS + 16 * s + 8 * h], kf[s], st);
      }
#pragma unroll
      for (int s = 0; s < C::DSV; ++s) {
        dpt = mfma32(*(const bf16x8*)&osm[buf][qrow * OS + 16 * s + 8 * h], vf[s], dpt);
      }
      if (need_mask) {
        // key visible iff key_pos <= query_pos: element i's query offset
        // 16*(i/8) + 4*(i%4) + 2*((i/4)%2) + h >= key_pos - qpos_s
        const int lim = (int)(wave_kpos0 + l32 - qpos_s) - h;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) < lim) st[i] = kNegInf;
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        f32x8 p, ds;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * t2 + e;
          p[e] = exp2_hw(st[i] * a.scale_log2);
          ds[e] = p[e] * dpt[i];
        }
        pb[t2] = to_bf16x8(p);
        dsb[t2] = to_bf16x8(ds);
      }
      // dV^T += dO^T P and dK^T += Q^T dS: step t2 holds accumulator rows 16*t2 + 4*h +
      // {0..3} and 16*t2 + 8 + 4*h + {0..3} in lane half h; dO^T / Q^T rows = 32*mt +
      // lane%32.
      // One flattened loop (dV tiles, then dK tiles), each step's transposed reads
      // issued while the previous step's products run.
      constexpr int NST = C::MTV + C::MT;
      auto trread = [&](int it, bf16x4 (&f)[2][2]) {
        const bool is_v = it < C::MTV;
        const int mt = is_v ? it : it - C::MTV;
        const int dcol = 32 * mt + 16 * (gg & 1) + 4 * (L & 3);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            // LDS row of accumulator row 16*t2 + 8*x + 4*(gg/2) + L/4
            const int r = qs * 32 + 16 * t2 + 4 * (L >> 2) + 2 * x + (gg >> 1);
            f[t2][x] = is_v ? lds_read_tr16(&osm[buf][r * OS + dcol]) : lds_read_tr16(&qsm[buf][r * QS + dcol]);
          }
      };
      bf16x4 fc[2][2], fn[2][2];
      trread(0, fc);
#pragma unroll
      for (int it = 0; it < NST; ++it) {
        if (it + 1 < NST) trread(it + 1, fn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          if (it < C::MTV)
            dvacc[it] = mfma32(cat(fc[t2][0], fc[t2][1]), pb[t2], dvacc[it]);
          else
            dkacc[it - C::MTV] = mfma32(cat(fc[t2][0], fc[t2][1]), dsb[t2], dkacc[it - C::MTV]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int x = 0; x < 2; ++x) fc[t2][x] = fn[t2][x];
      }
    }
  };

  load_tile(0, 0);
  store_rows(0);
  wait_vmem();
  __syncthreads();
  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    // the other buffer was last read before the previous barrier
    if (n + 1 < ntiles) load_tile(n + 1, buf ^ 1);
    compute_tile(buf, a.q_pos0 + tile_row0(n));
    if (n + 1 < ntiles) store_rows(buf ^ 1);
    wait_vmem();
    __syncthreads();
  }

  if (my_key < a.Sk) {
    float* dkp = a.dk + (kvh + my_key) * DQK;
    float* dvp = a.dv + (kvh + my_key) * DV;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * mt + 8 * g4 + 4 * h;
        f32x4 cur = *(const f32x4*)(dkp + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[e] = fmaf(a.scale, dkacc[mt][4 * g4 + e], cur[e]);
        *(f32x4*)(dkp + d) = cur;
      }
#pragma unroll
    for (int mt = 0; mt < C::MTV; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * mt + 8 * g4 + 4 * h;
        f32x4 cur = *(const f32x4*)(dvp + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[e] += dvacc[mt][4 * g4 + e];
        *(f32x4*)(dvp + d) = cur;
      }
  }
}

// ---- launchers ------------------------------------------------------------------------
hipError_t bwd_delta(const __bf16* o, const __bf16* dout, float* delta, long long rows, int Dv, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long long grid = (rows + 15) / 16;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)grid), dim3(256), 0, st, o, dout, delta, rows, Dv);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t bwd_launch(BwdArgs a, hipStream_t st) {
  using CK = BCfg<DQK, DV, kBwdWaves>;
  using CQ = BCfg<DQK, DV, kBwdWaves>;
  // dK, dV first: one workgroup per CK::ROWS keys of a (batch, KV head)
  BwdArgs b = a;
  b.n_tiles = (a.Sk + CK::ROWS - 1) / CK::ROWS;
  long long grid = 8 * (((long long)a.B * a.Hkv * b.n_tiles + 7) / 8);   // whole rounds of the 8 XCDs
  if (grid > 0x7ffffff0LL) return hipErrorInvalidValue;
  if (grid > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<DQK, DV, kBwdWaves>), dim3((unsigned)grid),
                       dim3(CK::THREADS), 0, st, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dQ: one workgroup per CQ::ROWS query rows of a (batch, head)
  b.n_tiles = (a.Sq + CQ::ROWS - 1) / CQ::ROWS;
  grid = 8 * (((long long)a.B * a.Hq * b.n_tiles + 7) / 8);
  if (grid > 0x7ffffff0LL) return hipErrorInvalidValue;
  if (grid > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, DV, kBwdWaves>), dim3((unsigned)grid), dim3(CQ::THREADS),
                       0, st, b);
  return hipGetLastError();
}

// Returns hipErrorInvalidValue when no kernel instance covers (dqk, dv).
hipError_t bwd_bf16(const BwdArgs& a, int dqk, int dv, hipStream_t st) {
  if (dqk == 128 && dv == 128) return bwd_launch<128, 128>(a, st);
  if (dqk == 64 && dv == 64) return bwd_launch<64, 64>(a, st);
  if (dqk == 192 && dv == 128) return bwd_launch<192, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
