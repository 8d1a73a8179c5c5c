// C ABI of libringattn.so: argument validation, kernel dispatch, per-thread error
// messages, and the host-side ring schedule. Every function validates all of its
// arguments before it enqueues anything, so an error return has launched nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/ringattn.h"
#include "common.hpp"

namespace ra {
hipError_t prefill_bf16(const PrefillArgs& a, int dqk, int dv, int step_mode, hipStream_t st);
hipError_t prefill_f32(const PrefillArgs& a, int dqk, int dv, int step_mode, hipStream_t st);
hipError_t lse_merge2(long long rows, int Dv, const float* o_a, const float* lse_a, const float* o_b,
                      const float* lse_b, float* o_out, float* lse_out, hipStream_t st);
hipError_t lse_merge_n(int out_bf16, long long rows, int n, int Dv, const float* o_parts,
                       const float* lse_parts, void* o_out, float* lse_out, hipStream_t st);
hipError_t decode_partial_bf16(const DecodeArgs& a, int d, int kv8, hipStream_t st);
hipError_t bwd_delta(const __bf16* o, const __bf16* dout, float* delta, long long rows, int Dv, hipStream_t st);
hipError_t bwd_bf16(const BwdArgs& a, int dqk, int dv, hipStream_t st);
hipError_t bwd_delta_f32(const float* o, const float* dout, float* delta, long long rows, int Dv, hipStream_t st);
hipError_t bwd_f32(const BwdArgs& a, int dqk, int dv, hipStream_t st);
size_t scratch_bytes();
hipError_t device_scratch(void** ptr);
}  // namespace ra

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return RA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bf16_dims_ok(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}
bool f32_dims_ok(int dqk, int dv) { return (dqk == 64 || dqk == 128) && (dv == 64 || dv == 128); }

// a per-(batch, head) slab must be addressable with 32-bit byte offsets
constexpr long long kMaxSlabBytes = 0x7fffffffLL;

int check_common(int dtype, int B, int Hq, int Hkv, int Dqk, int Dv, float scale) {
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_EINVAL, "dtype must be RA_F32 or RA_BF16");
  if (B <= 0 || Hq <= 0 || Hkv <= 0) return fail(RA_EINVAL, "B, Hq, Hkv must be positive");
  if (Hq % Hkv != 0) return fail(RA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Dqk <= 0 || Dv <= 0) return fail(RA_EINVAL, "head dims must be positive");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(RA_EINVAL, "scale must be finite and > 0");
  const bool dims = dtype == RA_BF16 ? bf16_dims_ok(Dqk, Dv) : f32_dims_ok(Dqk, Dv);
  if (!dims)
    return fail(RA_EUNSUPPORTED, "no %s kernel for (Dqk, Dv) = (%d, %d)", dtype == RA_BF16 ? "bf16" : "fp32",
                Dqk, Dv);
  return RA_OK;
}

// rows * d * esize <= 2^31 - 1, compared without forming the product (rows can be a
// product of two ints itself)
int check_slab(long long rows, int d, int esize, const char* name) {
  if (rows > kMaxSlabBytes / ((long long)d * esize))
    return fail(RA_EUNSUPPORTED, "%s: a per-head slab of %lld rows x %d exceeds 2^31 bytes", name, rows, d);
  return RA_OK;
}

}  // namespace

extern "C" {

int ra_abi_version(void) { return RA_ABI_VERSION; }

const char* ra_last_error(void) { return g_err.c_str(); }

int ra_ring_schedule(int P, int i, int causal, int* kv_block, int* kind) {
  if (P <= 0 || i < 0 || i >= P || !kv_block || !kind) {
    fail(RA_EINVAL, "ra_ring_schedule: need P > 0, 0 <= i < P and non-null outputs");
    return -RA_EINVAL;
  }
  for (int s = 0; s < P; ++s) {
    const int j = ((i - s) % P + P) % P;
    kv_block[s] = j;
    kind[s] = !causal ? 2 : (j > i ? 0 : (j == i ? 1 : 2));
  }
  ok();
  return P;
}

int ra_ring_schedule_striped(int P, int i, int causal, int* kv_block, int* kind) {
  if (P <= 0 || i < 0 || i >= P || !kv_block || !kind) {
    fail(RA_EINVAL, "ra_ring_schedule_striped: need P > 0, 0 <= i < P and non-null outputs");
    return -RA_EINVAL;
  }
  for (int s = 0; s < P; ++s) {
    kv_block[s] = ((i - s) % P + P) % P;
    kind[s] = causal ? 1 : 2;   // every block is a masked triangle under a causal mask
  }
  ok();
  return P;
}

}  // extern "C"

namespace {

int ring_fwd(const char* name, int striped, int dtype, const void* q, const void* k, const void* v, void* o,
             float* lse, int B, int Hq, int Hkv, int Sp, int P, int q_part0, int nq, int Dqk, int Dv,
             float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return fail(RA_EINVAL, "%s: null pointer", name);
  if (int r = check_common(dtype, B, Hq, Hkv, Dqk, Dv, scale)) return r;
  if (Sp <= 0 || P <= 0 || nq <= 0) return fail(RA_EINVAL, "Sp, P, nq must be positive");
  if (q_part0 < 0 || (long long)q_part0 + nq > P)
    return fail(RA_EINVAL, "query partitions %d..%d outside the ring of %d", q_part0, q_part0 + nq - 1, P);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(RA_EINVAL, "pointers must be 16-byte aligned");
  const int es = dtype == RA_BF16 ? 2 : 4;
  const long long kv_rows = (long long)P * Sp, q_rows = (long long)nq * Sp;
  if (int r = check_slab(kv_rows, Dqk > Dv ? Dqk : Dv, es, "k/v")) return r;
  if (int r = check_slab(q_rows, Dqk > Dv ? Dqk : Dv, es, "q/o")) return r;
  ra::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.q_rows = (int)q_rows;
  a.kv_rows = (int)kv_rows;
  a.Sp = Sp;
  a.P = P;
  a.q_part0 = q_part0;
  a.nq = nq;
  a.scale_log2 = scale * ra::kLog2e;
  a.causal = causal ? 1 : 0;
  a.striped = striped;
  hipStream_t st = (hipStream_t)stream;
  const hipError_t e = dtype == RA_BF16 ? ra::prefill_bf16(a, Dqk, Dv, 0, st) : ra::prefill_f32(a, Dqk, Dv, 0, st);
  return hip_status(e, name);
}

}  // namespace

extern "C" {

int ra_ring_attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Sp, int P, int q_part0, int nq, int Dqk, int Dv, float scale,
                     int causal, void* stream) {
  return ring_fwd("ra_ring_attn_fwd", 0, dtype, q, k, v, o, lse, B, Hq, Hkv, Sp, P, q_part0, nq, Dqk, Dv, scale,
                  causal, stream);
}

int ra_ring_attn_fwd_striped(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Sp, int P, int q_part0, int nq, int Dqk, int Dv,
                             float scale, int causal, void* stream) {
  return ring_fwd("ra_ring_attn_fwd_striped", 1, dtype, q, k, v, o, lse, B, Hq, Hkv, Sp, P, q_part0, nq, Dqk,
                  Dv, scale, causal, stream);
}

int ra_block_attn_step(int dtype, const void* q, long long q_pos0, int Sq, const void* k_blk, const void* v_blk,
                       long long k_pos0, int Sk, int B, int Hq, int Hkv, int Dqk, int Dv, float scale, int causal,
                       float* o_acc, float* lse_acc, void* stream) {
  if (!q || !k_blk || !v_blk || !o_acc || !lse_acc) return fail(RA_EINVAL, "ra_block_attn_step: null pointer");
  if (int r = check_common(dtype, B, Hq, Hkv, Dqk, Dv, scale)) return r;
  if (Sq <= 0 || Sk <= 0) return fail(RA_EINVAL, "Sq and Sk must be positive");
  if (q_pos0 < 0 || k_pos0 < 0) return fail(RA_EINVAL, "positions must be non-negative");
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o_acc) || !aligned16(lse_acc))
    return fail(RA_EINVAL, "pointers must be 16-byte aligned");
  const int es = dtype == RA_BF16 ? 2 : 4;
  if (int r = check_slab(Sk, Dqk > Dv ? Dqk : Dv, es, "k/v")) return r;
  if (int r = check_slab(Sq, Dqk > Dv ? Dqk : Dv, 4, "q/o_acc")) return r;
  ra::PrefillArgs a{};
  a.q = q;
  a.k = k_blk;
  a.v = v_blk;
  a.o_acc = o_acc;
  a.lse_acc = lse_acc;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.q_rows = Sq;
  a.kv_rows = Sk;
  a.q_pos0 = q_pos0;
  a.k_pos0 = k_pos0;
  a.Sk = Sk;
  a.nq = 1;
  a.P = 1;
  a.scale_log2 = scale * ra::kLog2e;
  a.causal = causal ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  const hipError_t e = dtype == RA_BF16 ? ra::prefill_bf16(a, Dqk, Dv, 1, st) : ra::prefill_f32(a, Dqk, Dv, 1, st);
  return hip_status(e, "ra_block_attn_step launch");
}

int ra_lse_merge(long long rows, int Dv, const float* o_a, const float* lse_a, const float* o_b,
                 const float* lse_b, float* o_out, float* lse_out, void* stream) {
  if (rows < 0 || Dv <= 0 || Dv % 4) return fail(RA_EINVAL, "need rows >= 0 and Dv a positive multiple of 4");
  if (rows == 0) return ok();
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return fail(RA_EINVAL, "ra_lse_merge: null pointer");
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out) || !aligned16(lse_a) || !aligned16(lse_b) ||
      !aligned16(lse_out))
    return fail(RA_EINVAL, "ra_lse_merge: pointers must be 16-byte aligned");
  return hip_status(ra::lse_merge2(rows, Dv, o_a, lse_a, o_b, lse_b, o_out, lse_out, (hipStream_t)stream),
                    "ra_lse_merge launch");
}

int ra_lse_merge_n(int out_dtype, long long rows, int n, int Dv, const float* o_parts, const float* lse_parts,
                   void* o_out, float* lse_out, void* stream) {
  if (out_dtype != RA_F32 && out_dtype != RA_BF16) return fail(RA_EINVAL, "out_dtype must be RA_F32 or RA_BF16");
  if (rows < 0 || n <= 0 || Dv <= 0 || Dv % 4) return fail(RA_EINVAL, "need rows >= 0, n > 0, Dv a positive multiple of 4");
  if (rows == 0) return ok();
  if (!o_parts || !lse_parts || !o_out || !lse_out) return fail(RA_EINVAL, "ra_lse_merge_n: null pointer");
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o_out) || !aligned16(lse_out))
    return fail(RA_EINVAL, "ra_lse_merge_n: pointers must be 16-byte aligned");
  return hip_status(ra::lse_merge_n(out_dtype == RA_BF16, rows, n, Dv, o_parts, lse_parts, o_out, lse_out,
                                    (hipStream_t)stream),
                    "ra_lse_merge_n launch");
}

}  // extern "C"

namespace {

// kv8: k_cache / v_cache hold fp8 e4m3 values, dequantised by k_scale / v_scale.
int splitkv_launch(int dtype, const void* q, const void* k_cache, const void* v_cache, int B, int Hq, int Hkv,
                   int L, int Dqk, int Dv, int n_splits, float scale, float* o_part, float* lse_part,
                   hipStream_t st, const char* who, int kv8 = 0, float k_scale = 1.f, float v_scale = 1.f) {
  if (!q || !k_cache || !v_cache || !o_part || !lse_part) return fail(RA_EINVAL, "%s: null pointer", who);
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_EINVAL, "dtype must be RA_F32 or RA_BF16");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || n_splits <= 0 || Dqk <= 0 || Dv <= 0)
    return fail(RA_EINVAL, "sizes must be positive");
  if (Hq % Hkv != 0) return fail(RA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (L % n_splits != 0) return fail(RA_EINVAL, "L (%d) must divide into n_splits (%d) equal chunks", L, n_splits);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(RA_EINVAL, "scale must be finite and > 0");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(RA_EINVAL, "k_scale and v_scale must be finite and > 0");
  if (!std::isfinite(scale * k_scale * ra::kLog2e))
    return fail(RA_EINVAL, "scale * k_scale overflows");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_part) || !aligned16(lse_part))
    return fail(RA_EINVAL, "%s: pointers must be 16-byte aligned", who);
  if (dtype != RA_BF16 || Dqk != Dv || (Dqk != 64 && Dqk != 128) || Hq / Hkv > 16)
    return fail(RA_EUNSUPPORTED, "split-KV decode supports bf16 with Dqk == Dv in {64, 128} and Hq/Hkv <= 16");
  if (int r = check_slab(L, Dqk, kv8 ? 1 : 2, "k/v cache")) return r;
  ra::DecodeArgs a{};
  a.q = (const __bf16*)q;
  a.k = k_cache;
  a.v = v_cache;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.L = L;
  a.n_splits = n_splits;
  a.Ls = L / n_splits;
  a.scale_log2 = scale * k_scale * ra::kLog2e;
  a.v_scale = v_scale;
  return hip_status(ra::decode_partial_bf16(a, Dqk, kv8, st), who);
}

}  // namespace

extern "C" {

int ra_splitkv_partial(int dtype, const void* q, const void* k_cache, const void* v_cache, int B, int Hq, int Hkv,
                       int L, int Dqk, int Dv, int n_splits, float scale, float* o_part, float* lse_part,
                       void* stream) {
  return splitkv_launch(dtype, q, k_cache, v_cache, B, Hq, Hkv, L, Dqk, Dv, n_splits, scale, o_part, lse_part,
                        (hipStream_t)stream, "ra_splitkv_partial");
}

int ra_splitkv_decode(int dtype, const void* q, const void* k_cache, const void* v_cache, int B, int Hq, int Hkv,
                      int L, int Dqk, int Dv, int n_splits, float scale, float* o_part, float* lse_part, void* o,
                      float* lse, void* stream) {
  if (!o || !lse) return fail(RA_EINVAL, "ra_splitkv_decode: null pointer");
  if (!aligned16(o) || !aligned16(lse)) return fail(RA_EINVAL, "pointers must be 16-byte aligned");
  if (int r = splitkv_launch(dtype, q, k_cache, v_cache, B, Hq, Hkv, L, Dqk, Dv, n_splits, scale, o_part,
                             lse_part, (hipStream_t)stream, "ra_splitkv_decode"))
    return r;
  const hipError_t e = ra::lse_merge_n(1, (long long)B * Hq, n_splits, Dv, o_part, lse_part, o, lse,
                                       (hipStream_t)stream);
  return hip_status(e, "ra_splitkv_decode merge launch");
}

int ra_splitkv_partial_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                           int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                           float* o_part, float* lse_part, void* stream) {
  return splitkv_launch(RA_BF16, q, k_cache, v_cache, B, Hq, Hkv, L, Dqk, Dv, n_splits, scale, o_part, lse_part,
                        (hipStream_t)stream, "ra_splitkv_partial_fp8", 1, k_scale, v_scale);
}

int ra_splitkv_decode_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                          int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                          float* o_part, float* lse_part, void* o, float* lse, void* stream) {
  if (!o || !lse) return fail(RA_EINVAL, "ra_splitkv_decode_fp8: null pointer");
  if (!aligned16(o) || !aligned16(lse)) return fail(RA_EINVAL, "pointers must be 16-byte aligned");
  if (int r = splitkv_launch(RA_BF16, q, k_cache, v_cache, B, Hq, Hkv, L, Dqk, Dv, n_splits, scale, o_part,
                             lse_part, (hipStream_t)stream, "ra_splitkv_decode_fp8", 1, k_scale, v_scale))
    return r;
  const hipError_t e = ra::lse_merge_n(1, (long long)B * Hq, n_splits, Dv, o_part, lse_part, o, lse,
                                       (hipStream_t)stream);
  return hip_status(e, "ra_splitkv_decode_fp8 merge launch");
}

int ra_splitkv_decode_noalloc(int dtype, const void* q, const void* k_cache, const void* v_cache, int B, int Hq,
                              int Hkv, int L, int Dqk, int Dv, int n_splits, float scale, void* o, float* lse,
                              void* stream) {
  const char* who = "ra_splitkv_decode_noalloc";
  if (!o || !lse) return fail(RA_EINVAL, "%s: null pointer", who);
  if (!aligned16(o) || !aligned16(lse)) return fail(RA_EINVAL, "%s: pointers must be 16-byte aligned", who);
  if (B <= 0 || Hq <= 0 || n_splits <= 0 || Dv <= 0) return fail(RA_EINVAL, "%s: sizes must be positive", who);
  // the partials [B, Hq, n_splits, Dv] fp32, then their LSEs [B, Hq, n_splits] fp32 at
  // the next 256-byte boundary, must fit the library's per-device scratch; each
  // product is bounded before the next factor joins it, so nothing wraps
  const unsigned long long cap = ra::scratch_bytes();
  unsigned long long parts = (unsigned long long)B * (unsigned long long)Hq;   // < 2^62
  if (parts <= cap) parts *= (unsigned long long)n_splits;                      // < 2^24 * 2^31
  const unsigned long long need =
      parts <= cap ? (parts * 4ULL * (unsigned long long)Dv + 255) / 256 * 256 + parts * 4 : ~0ULL;
  if (need > cap)
    return fail(RA_EINVAL, "%s: the partials of B %d x Hq %d x n_splits %d (Dv %d) do not fit the %zu bytes "
                "of scratch (B * Hq * n_splits * (Dv + 1) * 4 plus alignment must stay within it)", who, B, Hq,
                n_splits, Dv, ra::scratch_bytes());
  const unsigned long long o_bytes = (parts * 4ULL * (unsigned long long)Dv + 255) / 256 * 256;
  // every other argument is validated by splitkv_launch before anything is enqueued;
  // check them here first too, so that a bad call never looks the scratch up
  if (!q || !k_cache || !v_cache) return fail(RA_EINVAL, "%s: null pointer", who);
  void* base = nullptr;
  if (const hipError_t e = ra::device_scratch(&base); e != hipSuccess) return hip_status(e, who);
  float* o_part = (float*)base;
  float* lse_part = (float*)((char*)base + o_bytes);
  if (int r = splitkv_launch(dtype, q, k_cache, v_cache, B, Hq, Hkv, L, Dqk, Dv, n_splits, scale, o_part,
                             lse_part, (hipStream_t)stream, who))
    return r;
  const hipError_t e = ra::lse_merge_n(1, (long long)B * Hq, n_splits, Dv, o_part, lse_part, o, lse,
                                       (hipStream_t)stream);
  return hip_status(e, "ra_splitkv_decode_noalloc merge launch");
}

int ra_attn_bwd_preprocess(int dtype, const void* o, const void* dout, long long rows, int Dv, float* delta,
                           void* stream) {
  if (!o || !dout || !delta) return fail(RA_EINVAL, "ra_attn_bwd_preprocess: null pointer");
  if (dtype != RA_F32 && dtype != RA_BF16) return fail(RA_EINVAL, "dtype must be RA_F32 or RA_BF16");
  if (rows < 0 || Dv <= 0 || Dv % 8 != 0) return fail(RA_EINVAL, "need rows >= 0 and Dv a positive multiple of 8");
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta))
    return fail(RA_EINVAL, "ra_attn_bwd_preprocess: pointers must be 16-byte aligned");
  const hipError_t e =
      dtype == RA_BF16 ? ra::bwd_delta((const __bf16*)o, (const __bf16*)dout, delta, rows, Dv, (hipStream_t)stream)
                       : ra::bwd_delta_f32((const float*)o, (const float*)dout, delta, rows, Dv, (hipStream_t)stream);
  return hip_status(e, "ra_attn_bwd_preprocess launch");
}

int ra_block_attn_bwd_step(int dtype, const void* q, const void* dout, const float* lse, const float* delta,
                           long long q_pos0, int Sq, const void* k_blk, const void* v_blk, long long k_pos0, int Sk,
                           int B, int Hq, int Hkv, int Dqk, int Dv, float scale, int causal, float* dq_acc,
                           float* dk_acc, float* dv_acc, void* stream) {
  if (!q || !dout || !lse || !delta || !k_blk || !v_blk || !dq_acc || !dk_acc || !dv_acc)
    return fail(RA_EINVAL, "ra_block_attn_bwd_step: null pointer");
  if (int r = check_common(dtype, B, Hq, Hkv, Dqk, Dv, scale)) return r;
  if (Sq <= 0 || Sk <= 0) return fail(RA_EINVAL, "Sq and Sk must be positive");
  if (q_pos0 < 0 || k_pos0 < 0) return fail(RA_EINVAL, "positions must be >= 0");
  if (!aligned16(q) || !aligned16(dout) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(dq_acc) ||
      !aligned16(dk_acc) || !aligned16(dv_acc) || !aligned16(lse) || !aligned16(delta))
    return fail(RA_EINVAL, "pointers must be 16-byte aligned");
  const int es = dtype == RA_BF16 ? 2 : 4;
  if (int r = check_slab(Sq, Dqk > Dv ? Dqk : Dv, es, "q/dout")) return r;
  if (int r = check_slab(Sk, Dqk > Dv ? Dqk : Dv, es, "k/v")) return r;
  ra::BwdArgs a{};
  a.q = q;
  a.k = k_blk;
  a.v = v_blk;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq_acc;
  a.dk = dk_acc;
  a.dv = dv_acc;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.q_pos0 = q_pos0;
  a.k_pos0 = k_pos0;
  a.scale = scale;
  a.scale_log2 = scale * ra::kLog2e;
  a.causal = causal ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  const hipError_t e = dtype == RA_BF16 ? ra::bwd_bf16(a, Dqk, Dv, st) : ra::bwd_f32(a, Dqk, Dv, st);
  return hip_status(e, "ra_block_attn_bwd_step launch");
}

}  // extern "C"
