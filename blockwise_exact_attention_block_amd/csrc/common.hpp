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

// The same read at a 32-bit LDS byte address.
__device__ __forceinline__ bf16x4 lds_read_tr16_at(unsigned addr) {
  lds_bf16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((RA_LDS lds_bf16x4_t*)(uintptr_t)addr);
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
// Buffer descriptor words of make_rsrc, as four scalars for inline asm.
__device__ __forceinline__ u32x4 raw_desc(const void* base, unsigned nbytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4 r;
  r[0] = (unsigned)p;
  r[1] = (unsigned)(p >> 32) & 0xffffu;   // stride 0
  r[2] = nbytes;
  r[3] = 0x00020000u;
  return r;
}
// 32-bit LDS byte address of a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(RA_LDS const void*)p;
}
// 16 bytes per lane from a raw buffer straight into LDS (buffer_load ... lds): lane
// i's bytes land at lds_base + 16 * i, whatever its global offset; lds_base is
// wave-uniform and goes through M0, which the asm declares clobbered. It is issued
// from asm so that the compiler does not hold its own LDS reads of other buffers
// behind it. The data is visible only after wait_vmem() on the issuing wave and a
// barrier.
// M0 is a reserved register for the compiler, which warns that it does not save
// such a register around an asm statement. It need not: what the clobber does is
// make the compiler write M0 again before its own next use of it (with the clobber
// it reloads M0 after the asm; without it, it would reuse the value it set
// earlier), so no value of the compiler's lives in M0 across this asm.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(unsigned lds_base, unsigned byte_off, u32x4 desc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(byte_off), "s"(desc) : "memory", "m0");
}
#pragma clang diagnostic pop
// Direct HBM -> LDS loads of a tile of ROWS consecutive global rows of ROW_BYTES bytes
// into LDS rows of LDS_STRIDE bytes (the row plus padding). The LDS tile is cut into
// 1 KB pieces, and piece j is written by one wave-wide lds_load16, whose lane i fills
// bytes [1024 j + 16 i, +16) of the tile. It fetches the 16 global bytes that belong
// there, or, for a slot in a row's padding, a duplicate of that row's first bytes
// (never read). Piece j goes to wave j % NW. The tile's LDS allocation is a whole
// number of KB (padded_tile_bytes); when ROWS * LDS_STRIDE is not, the last piece's
// slots past the tile fetch the following global rows (clamped like every offset)
// into that slack, which is never read.
constexpr int padded_tile_bytes(int rows, int lds_stride) { return (rows * lds_stride + 1023) / 1024 * 1024; }
template <int ROWS, int ROW_BYTES, int LDS_STRIDE, int NW>
struct PaddedTileDma {
  static constexpr int PIECES = padded_tile_bytes(ROWS, LDS_STRIDE) / 1024;
  static constexpr int PER_WAVE = (PIECES + NW - 1) / NW;
  static_assert(LDS_STRIDE % 16 == 0 && ROW_BYTES % 16 == 0 && LDS_STRIDE - ROW_BYTES <= ROW_BYTES, "layout");
  unsigned off[PER_WAVE];   // per lane: global byte offset inside the tile, per piece
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int p = (wave + q * NW) * 1024 + lane * 16;
      const int row = p / LDS_STRIDE, within = p - row * LDS_STRIDE;
      off[q] = (unsigned)(row * ROW_BYTES + (within < ROW_BYTES ? within : within - ROW_BYTES));
    }
  }
  // wave: wave-uniform index; gbase: global byte offset of the tile's first row;
  // glast: last valid 16-byte offset of the buffer (rows past it re-read it).
  __device__ __forceinline__ void issue(int wave, unsigned lds_tile, unsigned gbase, unsigned glast,
                                        u32x4 desc) const {
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      const int j = wave + q * NW;
      if (j < PIECES) lds_load16(lds_tile + (unsigned)j * 1024u, min(gbase + off[q], glast), desc);
    }
  }
};
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima). As a builtin, the
// compiler's own wait tracking sees it, so it adds no waits of its own later on.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// Non-temporal 16-byte load (cache policy nt): for data read exactly once, such as
// a KV cache streamed by decode. (8-byte loads with this policy measured slower.)
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0);
  return make_uint2(v[0], v[1]);
}

// Four fp8 e4m3 values (OCP format, one 32-bit word) to four bf16, exactly: every
// e4m3 value is a bf16 value. v_cvt_scalef32_pk_bf16_fp8 converts the low or high
// 16 bits of the word, with a scale of 1.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(unsigned w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi));
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
  int striped;        // 0: partition p = tokens p*Sp .. p*Sp+Sp-1; 1: tokens p, p+P, p+2P, ...
  // step mode
  long long q_pos0, k_pos0;
  int Sk;
  int n_qtiles;       // query tiles per (b, h) and per query partition
  float scale_log2;   // softmax scale * log2(e)
  int causal;
};

// Key-tile schedule of one query tile in ring mode: the KV blocks in ring order,
// block (i - s) mod P at step s, each cut into tiles of BK keys.
//   * contiguous layout (partition p holds global tokens p*Sp .. p*Sp + Sp - 1),
//     causal: the own block i first, only up to the query tile's last row, then
//     the full blocks i-1 .. 0; blocks after i hold only future keys and are not
//     visited. Tile positions are global token positions.
//   * striped layout (partition p holds global tokens p, p + P, p + 2P, ...),
//     causal: key c of block j is visible to local query row r iff
//     c*P + j <= r*P + i, i.e. c + [j > i] <= r. Every block is visited up to the
//     query tile's last row, and masks compare "virtual" positions: the local row
//     for a query, local index + [j > i] for a key.
//   * without a causal mask both layouts visit every tile of every block.
// last_local: local index of the query tile's last row inside its partition.
struct RingTiles {
  int i, P, Sp, BK, n_full, na, nb, ntiles;
  bool causal, striped;
  __device__ __forceinline__ void init(int i_, int P_, int Sp_, int BK_, bool causal_, bool striped_,
                                       int last_local) {
    i = i_; P = P_; Sp = Sp_; BK = BK_; causal = causal_; striped = striped_ && causal_;
    n_full = (Sp + BK - 1) / BK;
    na = last_local / BK + 1;                                 // tiles up to the last row
    nb = last_local >= 1 ? (last_local - 1) / BK + 1 : 0;    // same, one key position later
    if (!causal)
      ntiles = P * n_full;
    else if (striped)
      ntiles = (i + 1) * na + (P - 1 - i) * nb;
    else
      ntiles = na + i * n_full;
  }
  // tile n -> first key row in the [P*Sp] block-major K/V slab, position of that
  // key (global, or virtual for the striped causal case) and valid keys (<= BK)
  __device__ __forceinline__ void tile(int n, int& row0, long long& pos0, int& nvalid) const {
    int j, tt, shift = 0;
    if (!causal) {
      const int s = n / n_full;
      tt = n - s * n_full;
      j = i - s;
      if (j < 0) j += P;
    } else if (striped) {
      if (n < (i + 1) * na) {
        const int s = n / na;
        tt = n - s * na;
        j = i - s;
      } else {
        const int r = n - (i + 1) * na;
        const int s = r / nb;
        tt = r - s * nb;
        j = P - 1 - s;          // steps i+1 .. P-1 visit blocks P-1 .. i+1
        shift = 1;
      }
    } else if (n < na) {
      j = i;
      tt = n;
    } else {
      const int r = n - na;
      const int s = 1 + r / n_full;
      j = i - s;
      tt = r - (s - 1) * n_full;
    }
    row0 = j * Sp + tt * BK;
    pos0 = striped ? (long long)(tt * BK + shift) : (long long)j * Sp + tt * BK;
    nvalid = min(BK, Sp - tt * BK);
  }
  // The same schedule walked one tile at a time, without divisions: block j, tile
  // tt of the ntt tiles taken from it, key shift of the striped causal case.
  struct Cursor {
    int j, tt, ntt, shift;
  };
  __device__ __forceinline__ Cursor start() const {
    Cursor c;
    c.j = i;
    c.tt = 0;
    c.ntt = causal ? na : n_full;
    c.shift = 0;
    return c;
  }
  // Moves to the next tile; only called while tiles remain.
  __device__ __forceinline__ void advance(Cursor& c) const {
    if (++c.tt < c.ntt) return;
    c.tt = 0;
    if (!causal) {
      c.j = (c.j == 0 ? P : c.j) - 1;
    } else if (!striped) {
      c.j -= 1;
      c.ntt = n_full;
    } else if (c.shift == 0 && c.j > 0) {
      c.j -= 1;
    } else if (c.shift == 0) {
      c.j = P - 1;          // steps i+1 .. P-1 visit blocks P-1 .. i+1, one key later
      c.ntt = nb;
      c.shift = 1;
    } else {
      c.j -= 1;
    }
  }
  __device__ __forceinline__ void at(const Cursor& c, int& row0, long long& pos0, int& nvalid) const {
    row0 = c.j * Sp + c.tt * BK;
    pos0 = striped ? (long long)(c.tt * BK + c.shift) : (long long)c.j * Sp + c.tt * BK;
    nvalid = min(BK, Sp - c.tt * BK);
  }
};

// Arguments of the backward kernels: one (query block, KV block) pair's gradient
// contributions, added into fp32 accumulators. BHSD layouts; lse / delta are the
// queries' full-row values saved by (or derived from) the forward pass.
struct BwdArgs {
  const void* q;      // [B, Hq, Sq, Dqk]
  const void* k;      // [B, Hkv, Sk, Dqk]
  const void* v;      // [B, Hkv, Sk, Dv]
  const void* dout;   // [B, Hq, Sq, Dv]
  const float* lse;   // [B, Hq, Sq]
  const float* delta; // [B, Hq, Sq]  rowsum(dO o O)
  float* dq;          // [B, Hq, Sq, Dqk]  += scale * dS K
  float* dk;          // [B, Hkv, Sk, Dqk] += scale * dS^T Q (summed over the group's heads)
  float* dv;          // [B, Hkv, Sk, Dv]  += P^T dO
  int B, Hq, Hkv, group, Sq, Sk;
  long long q_pos0, k_pos0;
  float scale, scale_log2;
  int causal;
  int n_tiles;        // launcher: query tiles (dQ kernel) or key tiles (dK/dV kernel) per head
};

// Arguments of the split-KV decode partial kernel.
struct DecodeArgs {
  const __bf16* q;   // [B, Hq, D]
  const void* k;     // [B, Hkv, L, D], bf16 or fp8 e4m3
  const void* v;     // [B, Hkv, L, D], bf16 or fp8 e4m3
  float* o_part;     // [B, Hq, n_splits, D]
  float* lse_part;   // [B, Hq, n_splits]
  int B, Hq, Hkv, G, L, n_splits, Ls;
  float scale_log2;  // softmax scale (times the K dequantisation scale) times log2(e)
  float v_scale;     // V dequantisation scale, applied to the normalised output
};

}  // namespace ra
