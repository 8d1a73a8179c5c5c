// Shared device helpers for the gfx950 kernels: vector types, MFMA wrappers,
// transposed LDS reads, exp2/log2 on the hardware transcendental unit, and the
// per-launch argument blocks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4_t;
#define RA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed 16-bit LDS read: inside each group of 16 lanes the lanes' 8-byte
// addresses form a 4-row x 16-column block (lane L reads row L/4, columns
// 4*(L%4)..+3); lane L receives column L of that block, rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  lds_bf16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((RA_LDS lds_bf16x4_t*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even fp32 -> bf16 of eight values.
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// max(v, v of the lane 32 apart), on every lane: v_permlane32_swap exchanges the
// two 32-lane halves, so each lane sees both values without an LDS round trip.
__device__ __forceinline__ float row_max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + nbytes): loads past the end return zero.
// base must be uniform across the wave. Word 3 selects 32-bit raw addressing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Arguments of one prefill launch (ring or single step). Element strides are in
// elements of the tensor's own dtype; all tensors are BHSD.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;            // ring: output in the input dtype
  float* lse;         // ring: output LSE
  float* o_acc;       // step: running fp32 state (in/out)
  float* lse_acc;     // step: running LSE (in/out)
  int B, Hq, Hkv, group;
  int q_rows;         // query rows per (b, h) in the q tensor
  int kv_rows;        // key rows per (b, kv head) in the k/v tensors
  // ring mode
  int Sp, P, q_part0, nq;
  // step mode
  long long q_pos0, k_pos0;
  int Sk;
  int n_qtiles;       // query tiles per (b, h) and per query partition
  float scale_log2;   // softmax scale * log2(e)
  int causal;
};

// Arguments of the split-KV decode partial kernel.
struct DecodeArgs {
  const __bf16* q;   // [B, Hq, D]
  const __bf16* k;   // [B, Hkv, L, D]
  const __bf16* v;   // [B, Hkv, L, D]
  float* o_part;     // [B, Hq, n_splits, D]
  float* lse_part;   // [B, Hq, n_splits]
  int B, Hq, Hkv, G, L, n_splits, Ls;
  float scale_log2;
};

}  // namespace ra
