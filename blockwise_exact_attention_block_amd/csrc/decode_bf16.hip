// Split-KV ("pass-Q") decode attention for gfx950: partial attention of one new
// query token per sequence over each contiguous chunk of its KV cache, giving a
// normalised partial output and its LSE per chunk (page "上下文并行 (CP) 收益评估
// 实验设计", §名词定义 pass-Q and §Decode). Reading the cache once is the whole cost
// (page "长上下文的第一性挑战", §KV 是 Decode 阶段的隐性瓶颈), so the kernel is built
// to stream K and V from HBM exactly once for all query heads of a KV group.
//
// Workgroup = (batch b, KV head g, split p), 4 waves. The split's keys are dealt to
// the waves in chunks of 32 keys (chunk c goes to wave c % 4), every wave running
// the same number of iterations (keys past the split are masked).
// Per chunk, on v_mfma_f32_16x16x32_bf16 with the G = Hq/Hkv heads as the 16-wide
// N dimension (heads >= G are zero queries):
//   * S^T = K Q^T: K comes straight from HBM into the A operand (lane = key,
//     8 consecutive d), Q^T sits in VGPRs for the whole kernel.
//   * online softmax per head (lane column): running max / exp-sum, rescale.
//   * O^T += V^T P^T: P^T is the S^T accumulator converted to bf16; V goes HBM ->
//     VGPR -> a wave-private LDS tile and is read back transposed with
//     ds_read_b64_tr_b16 in the accumulator's key order. The tile is private, so
//     the waves need no barrier until the merge (a per-chunk workgroup barrier
//     measured 3 % slower on an fp8 cache).
// The four waves' states are merged through LDS at the end. The cache is read with
// 16-byte loads in the non-temporal policy: every byte is read once, and streaming
// it that way measured faster. With an fp8 cache a lane's K fragments (8 values
// per MFMA step) are taken from one contiguous run of the row, d = 8 * DSTEP * gg
// + 8 s (the query fragments use the same mapping), so that they too come in
// 16-byte loads.
//
// FP8 KV (KV8): the cache holds e4m3 values with one dequantisation scale for K and
// one for V (1 byte per value, [CH] §挑战 2 KV-size equation with b = 1). K and V
// are read at half the bytes and converted exactly to bf16 in registers, so the
// products are the bf16 ones; the K scale is folded into the score scale and the
// V scale multiplies the normalised output.
#include "common.hpp"

namespace ra {

template <int D, bool KV8>
__global__ void __launch_bounds__(256)
decode_partial_kernel(DecodeArgs a) {
  constexpr int NW = 4, CK = 32;        // waves, keys per wave-chunk
  constexpr int EB = KV8 ? 1 : 2;       // bytes per cached value
  constexpr int VS = D + 16;            // padded LDS row (keys are rows)
  constexpr int DSTEP = D / 32;         // K-dim steps of the S MFMA
  constexpr int DM = D / 16;            // 16-row output tiles
  constexpr int VCH = CK * D / 8 / 64;  // 16-byte V chunks per lane per chunk (bf16)
  constexpr int VCH8 = CK * D / 16 / 64;  // 16-byte V chunks per lane per chunk (fp8)
  constexpr int VBUF = CK * VS;         // elements of one wave's V tile
  __shared__ __attribute__((aligned(16))) __bf16 vbuf[NW][2][VBUF];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L16 = lane & 15, gg = lane >> 4;
  const int split = blockIdx.x % a.n_splits;
  const int bg = blockIdx.x / a.n_splits;   // b * Hkv + g
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int key_begin = split * a.Ls;

  const size_t slab = (size_t)a.L * D;
  const auto krs = make_rsrc((const char*)a.k + (size_t)bg * slab * EB, (unsigned)(slab * EB));
  const auto vrs = make_rsrc((const char*)a.v + (size_t)bg * slab * EB, (unsigned)(slab * EB));

  // Q^T fragments: lane column = head L16 of the group, k-slots 8*gg + j of step s
  bf16x8 qf[DSTEP];
  {
    const int head = L16;
    const bool valid = head < a.G;
    const __bf16* qp = a.q + ((size_t)b * a.Hq + (size_t)g * a.G + (valid ? head : 0)) * D;
#pragma unroll
    for (int s = 0; s < DSTEP; ++s) {
      if (valid)
        qf[s] = *(const bf16x8*)(qp + (KV8 ? 8 * DSTEP * gg + 8 * s : 32 * s + 8 * gg));
      else
        qf[s] = bf16x8{};
    }
  }

  const int nchunks = (a.Ls + CK - 1) / CK;
  const int iters = (nchunks + NW - 1) / NW;

  uint4 kreg[2][DSTEP], vreg[VCH];       // bf16 cache
  uint4 kreg8[2][DSTEP / 2];              // fp8 cache: 16 values of one K row (two steps)
  uint4 vreg8[VCH8];                      // fp8 cache: 16 values of one V row
  auto load_chunk = [&](int it) {
    const int key0 = key_begin + (it * NW + wave) * CK;   // may lie past the split: masked later
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (KV8) {
        // fp8: the lane's DSTEP fragments are one run of 8 * DSTEP bytes
#pragma unroll
        for (int j = 0; j < DSTEP / 2; ++j)
          kreg8[kt][j] = buf_load16_nt(krs, (unsigned)((key0 + 16 * kt + L16) * D + 8 * DSTEP * gg + 16 * j));
      } else {
#pragma unroll
        for (int s = 0; s < DSTEP; ++s)
          kreg[kt][s] = buf_load16_nt(krs, (unsigned)((key0 + 16 * kt + L16) * D + 32 * s + 8 * gg) * 2u);
      }
    }
    if (KV8) {
#pragma unroll
      for (int c = 0; c < VCH8; ++c) {
        const int e = c * 64 + lane;
        const int row = e / (D / 16), col = e % (D / 16);
        vreg8[c] = buf_load16_nt(vrs, (unsigned)((key0 + row) * D + col * 16));
      }
    } else {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int e = c * 64 + lane;
        const int row = e / (D / 8), col = e % (D / 8);
        vreg[c] = buf_load16_nt(vrs, (unsigned)((key0 + row) * D + col * 8) * 2u);
      }
    }
  };

  float m = kNegInf, l = 0.f;
  f32x4 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x4{};

  if (iters > 0) load_chunk(0);
  for (int it = 0; it < iters; ++it) {
    const int buf = it & 1;
    __bf16* vb = vbuf[wave][buf];
    if (KV8) {
#pragma unroll
      for (int c = 0; c < VCH8; ++c) {
        const int e = c * 64 + lane;
        const int row = e / (D / 16), col = e % (D / 16);
        const uint2 b0 = fp8x4_to_bf16x4(vreg8[c].x), b1 = fp8x4_to_bf16x4(vreg8[c].y);
        const uint2 b2 = fp8x4_to_bf16x4(vreg8[c].z), b3 = fp8x4_to_bf16x4(vreg8[c].w);
        *(uint4*)&vb[row * VS + col * 16] = make_uint4(b0.x, b0.y, b1.x, b1.y);
        *(uint4*)&vb[row * VS + col * 16 + 8] = make_uint4(b2.x, b2.y, b3.x, b3.y);
      }
    } else {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int e = c * 64 + lane;
        const int row = e / (D / 8), col = e % (D / 8);
        *(uint4*)&vb[row * VS + col * 8] = vreg[c];
      }
    }
    uint4 kcur[2][DSTEP];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < DSTEP; ++s) {
        if (KV8) {
          const uint4 w = kreg8[kt][s / 2];
          const uint2 lo = fp8x4_to_bf16x4(s % 2 ? w.z : w.x), hi = fp8x4_to_bf16x4(s % 2 ? w.w : w.y);
          kcur[kt][s] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          kcur[kt][s] = kreg[kt][s];
        }
      }
    if (it + 1 < iters) load_chunk(it + 1);
    // No barrier: the V tile is private to the wave, and one wave's LDS operations
    // complete in the order they are issued, so the reads below see these writes
    // and the next chunk's writes (to the other buffer) come after them. The waves
    // run at their own pace until the merge.

    const int key0 = (it * NW + wave) * CK;   // relative to the split
    f32x4 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x4{};
#pragma unroll
      for (int s = 0; s < DSTEP; ++s) sacc[kt] = mfma16(__builtin_bit_cast(bf16x8, kcur[kt][s]), qf[s], sacc[kt]);
    }
    // keys of the chunk past the split's end see -inf
    const int lim = a.Ls - key0 - 4 * gg;   // keys 16*kt + i (+4*gg) must be < Ls - key0
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sv = (16 * kt + i) < lim ? sacc[kt][i] : kNegInf;
        sacc[kt][i] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mnew = fmaxf(m, mx * a.scale_log2);
    const float muse = mnew == kNegInf ? 0.f : mnew;
    const float alpha = exp2_hw(m - muse);
    m = mnew;
    float rs = 0.f;
    f32x8 pv;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_hw(fmaf(sacc[kt][i], a.scale_log2, -muse));
        pv[4 * kt + i] = p;
        rs += p;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    const bf16x8 pb = to_bf16x8(pv);
    // P^T slot (gg, j) holds key 16*(j/4) + 4*gg + j%4; the transposed V reads
    // deliver the same keys for output columns 16*dm + L16.
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
      const int dcol = 16 * dm + 4 * (L16 & 3);
      bf16x4 h2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int key = 16 * x + 4 * gg + (L16 >> 2);
        h2[x] = lds_read_tr16(&vb[key * VS + dcol]);
      }
      oacc[dm] = mfma16(cat(h2[0], h2[1]), pb, oacc[dm]);
    }
  }

  // ---- merge the four waves' states ---------------------------------------------
  __syncthreads();  // V tiles no longer read: reuse that LDS
  float* sm = (float*)&vbuf[0][0][0];            // [NW][16] running max (log2 domain)
  float* sl = sm + NW * 16;                      // [NW][16] exp-sums
  float* so = sl + NW * 16;                      // [NW][16][D] unnormalised outputs
  const float lsum = l + shfl_xor_f(l, 16);
  const float lt = lsum + shfl_xor_f(lsum, 32);
  if (gg == 0) {
    sm[wave * 16 + L16] = m;
    sl[wave * 16 + L16] = lt;
  }
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[(wave * 16 + L16) * D + 16 * dm + 4 * gg + i] = oacc[dm][i];
  __syncthreads();
  for (int e = threadIdx.x; e < a.G * D; e += 256) {
    const int head = e / D, d = e - head * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * 16 + head]);
    const float Ms = M == kNegInf ? 0.f : M;
    float lsum_all = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2_hw(sm[w * 16 + head] - Ms);
      lsum_all += f * sl[w * 16 + head];
      o += f * so[(w * 16 + head) * D + d];
    }
    const size_t hq = (size_t)b * a.Hq + (size_t)g * a.G + head;
    const size_t pi = hq * a.n_splits + split;
    a.o_part[pi * D + d] = lsum_all > 0.f ? o / lsum_all * a.v_scale : 0.f;
    if (d == 0) a.lse_part[pi] = lsum_all > 0.f ? (Ms + log2_hw(lsum_all)) * kLn2 : kNegInf;
  }
}

// kv8: the cache is fp8 e4m3 (1 byte per value) instead of bf16.
hipError_t decode_partial_bf16(const DecodeArgs& a, int d, int kv8, hipStream_t st) {
  const long long grid = (long long)a.B * a.Hkv * a.n_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), blk(256);
  if (d == 128 && !kv8)
    hipLaunchKernelGGL((decode_partial_kernel<128, false>), g, blk, 0, st, a);
  else if (d == 64 && !kv8)
    hipLaunchKernelGGL((decode_partial_kernel<64, false>), g, blk, 0, st, a);
  else if (d == 128 && kv8)
    hipLaunchKernelGGL((decode_partial_kernel<128, true>), g, blk, 0, st, a);
  else if (d == 64 && kv8)
    hipLaunchKernelGGL((decode_partial_kernel<64, true>), g, blk, 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ra
