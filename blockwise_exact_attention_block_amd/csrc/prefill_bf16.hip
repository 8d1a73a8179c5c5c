// bf16 blockwise exact attention for gfx950 (MI355X): ring prefill and single ring
// step, on v_mfma_f32_32x32x16_bf16.
//
// What is computed: for every query row, exact softmax(scale * q K^T) V over the
// visible keys of a sequence of KV blocks, visited one block at a time. Each KV tile
// updates the row's running maximum and exp-sum, rescales the output accumulator
// and adds the tile's contribution, so the result is the one-shot softmax
// (page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条超长序列",
// §"最容易被忽略的细节：不同 Block 的 Attention 结果不能直接相加"). In ring mode the
// blocks are taken in ring order, block (i - s) mod P at step s, with causal block
// skipping and an element-wise mask on the diagonal block only (same page, §"KV 在
// Ring 中如何流动"). In step mode the running state arrives as a normalised fp32
// output plus LSE and leaves in the same form (page "LLM长文本推理Ring Attention环形
// 注意力机制实现与优化", §Ring Attention实现代码与通信重叠).
//
// Data flow per workgroup (NW waves, each owning NQ x 32 query rows):
//   * Q rows of the wave are loaded once into VGPRs as the B operand of
//     S^T = K Q^T, so each lane owns one query column of the score tile and the row
//     maximum / sum are in-lane plus one exchange with the lane 32 apart
//     (v_permlane32_swap).
//   * K and V tiles of BK keys are double buffered in LDS and go straight from HBM
//     into it (buffer_load ... lds, one tile ahead). At D = 128 and at D_qk = 192,
//     D_v = 128 the tiles are 128 keys of unpadded rows whose 16-byte chunks are
//     XOR-swizzled against bank conflicts (two such tiles take 128 KB and exactly
//     160 KB of LDS); D = 64 keeps 128-key tiles of rows padded against bank
//     conflicts.
//   * One online-softmax update per tile: S^T for all BK keys (BK/32 accumulator
//     blocks, exact fp32 scores of the bf16 inputs), the tile's row max, then
//     P = exp2(scale * log2(e) * s - m) and PV. Each row carries a reference shift m
//     (exp2 domain). It is set to the row's max on its first visible tile. After
//     that it moves only when a scaled score of the tile exceeds it by more than
//     kLazyShift; then the accumulator and the exp-sum are rescaled once. Otherwise
//     P <= 2^kLazyShift, far from fp32 and bf16 limits. Softmax does not depend on
//     the shift, so the result is the same for any m.
//   * P^T for O^T += V^T P^T is taken straight from the S^T accumulator registers
//     (converted to bf16, round to nearest even). V^T operands come from the
//     natural [key][d] LDS tile through ds_read_b64_tr_b16, with the key order
//     inside each 16-key step matching the accumulator's row order.
//   * The output accumulator O^T keeps one query per lane column, so rescaling by
//     the shift's correction is a per-lane multiply.
#include "common.hpp"
#include <type_traits>

namespace ra {

// Query tiles per block when workgroups are dealt to the XCDs in blocks (see the
// workgroup mapping in prefill_bf16_kernel).
constexpr int kXcdTiles = 4;

enum { MODE_RING = 0, MODE_STEP = 1 };

// Largest lead (log2 units) of a score over its row's reference shift before the
// shift is moved: P stays below 2^8 between moves.
constexpr float kLazyShift = 8.0f;

template <int DQK, int DV, int NQ, int NW, int SPLIT>
struct PCfg {
  // SPLIT = 1: 128 keys per tile, all through one online-softmax update. Two
  // double-buffered tiles take 128 KB of LDS at D = 128, exactly 160 KB at
  // D_qk = 192 / D_v = 128 (unpadded rows) and 84 KB at D = 64 (padded rows).
  // SPLIT = 2: two key streams of 64-key tiles, each double-buffered (the same LDS).
  static constexpr int BK = SPLIT == 1 ? 128 : 64;
  static constexpr int THREADS = NW * 64;
  static constexpr int NWS = NW / SPLIT;              // waves per key stream
  static constexpr int BQ = NWS * NQ * 32;            // query rows per workgroup
  // D = 128 (DMA) and D_qk = 192 (DMAW): unpadded rows with an XOR swizzle of
  // 16-byte chunks. D = 64: rows padded so that consecutive K rows (16-byte reads)
  // and V rows (transposed 8-byte reads) start on different banks. Either way each
  // lane's reads are a per-lane base plus a compile-time offset.
  static constexpr bool DMA = DQK == 128 && DV == 128;     // one 256-byte row layout for K and V
  static constexpr bool DMAW = DQK == 192 && DV == 128;    // 384-byte K rows, 256-byte V rows
  static constexpr int KS = (DMA || DMAW) ? DQK : DQK + 8;
  static constexpr int VS = (DMA || DMAW) ? DV : DV + 32;
  static constexpr int K_TILE = padded_tile_bytes(BK, KS * 2) / 2;   // elements, whole KB
  static constexpr int V_TILE = padded_tile_bytes(BK, VS * 2) / 2;
  static_assert(2 * SPLIT * (K_TILE + V_TILE) * 2 <= 160 * 1024, "two tiles of K and V per stream must fit in LDS");
  static constexpr int DS = DQK / 16;                 // MFMA k-steps along D_qk
  static constexpr int MT = DV / 32;                  // 32-row output tiles along D_v
};

struct TileRef {
  int row0;        // first key row of the tile inside the (b, kv head) slab
  long long pos0;  // global token position of that key
  int nvalid;      // keys of the tile that exist (<= BK)
};

template <int DQK, int DV, int NQ, int NW, int MODE, int SPLIT>
__global__ void __launch_bounds__(NW * 64)
prefill_bf16_kernel(PrefillArgs a) {
  using C = PCfg<DQK, DV, NQ, NW, SPLIT>;
  constexpr int BK = C::BK, NWS = C::NWS;
  __shared__ __attribute__((aligned(16))) __bf16 ks[2 * SPLIT][C::K_TILE];
  __shared__ __attribute__((aligned(16))) __bf16 vs[2 * SPLIT][C::V_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // SPLIT = 2: waves 0 .. NWS-1 are key stream 0, the rest stream 1; both streams
  // cover the same query rows (row group = wave index within the stream)
  const int stream = SPLIT == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / NWS;   // wave-uniform
  const int wave = (tid >> 6) - stream * NWS;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // Workgroup -> (batch, head, query partition, query tile), XCD-aware. Workgroups
  // are dealt to the 8 XCDs round-robin, so XCD x runs ids x, x+8, ...; the work
  // list is ordered (batch, KV head, query tile, query head of the group), the
  // heaviest causal tiles of a KV head first. When the KV heads (times batch) are a
  // multiple of 8, XCD x takes the x-th contiguous eighth of the list: whole KV
  // heads, so the ~32 workgroups it runs at once are the query heads of one KV head
  // on a few adjacent query tiles, streaming the same K/V blocks through its L2.
  // Otherwise an eighth would hold part of a KV head's tiles (with two KV heads, XCD
  // 0 its heaviest quarter and XCD 3 its lightest), so the list is cut into blocks
  // of kXcdTiles query tiles (with all query heads of the group), dealt in rounds of
  // eight, one block per XCD, in serpentine order (round r deals blocks 8 r .. 8 r + 7
  // to XCDs 0 .. 7 when r is even and 7 .. 0 when it is odd): as the weights of
  // heavy-first causal tiles fall about linearly, every XCD's sum comes out even,
  // and its concurrent workgroups still read one KV head.
  const int tiles_per_head = (MODE == MODE_RING ? a.nq : 1) * a.n_qtiles;
  const int n_items = a.B * a.Hq * tiles_per_head;
  int u;
  if (((a.B * a.Hkv) & 7) == 0) {
    const int per_xcd = (n_items + 7) >> 3;
    u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  } else {
    const int bs = kXcdTiles * a.group;   // items per dealt block
    const int x = (int)(blockIdx.x & 7), j = (int)(blockIdx.x >> 3);
    const int r = j / bs;                 // the round: one block per XCD
    u = (8 * r + ((r & 1) ? 7 - x : x)) * bs + j % bs;
  }
  if (u >= n_items) return;  // padding of the last round: no work, no barrier
  const int w = u % a.group;
  const int rest = u / a.group;
  const int gt = tiles_per_head - 1 - rest % tiles_per_head;
  const int bg = rest / tiles_per_head;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int hq = g * a.group + w;
  const int bh = b * a.Hq + hq;
  int part = 0, qt = gt;
  if (MODE == MODE_RING) {
    part = gt / a.n_qtiles;
    qt = gt - part * a.n_qtiles;
  }

  int row_base, row_end;
  long long pos_base;
  if (MODE == MODE_RING) {
    row_base = part * a.Sp + qt * C::BQ;
    row_end = part * a.Sp + a.Sp;
    // striped causal: virtual query position = local row (see RingTiles)
    pos_base = (a.causal && a.striped ? 0LL : (long long)(a.q_part0 + part) * a.Sp) + qt * C::BQ;
  } else {
    row_base = qt * C::BQ;
    row_end = a.q_rows;
    pos_base = a.q_pos0 + row_base;
  }
  const int last_row = min(row_base + C::BQ, row_end) - 1;
  const long long last_pos = pos_base + (last_row - row_base);

  // the query slab as a raw buffer (rows past it read as zero); K / V slabs of one
  // (batch, KV head) start at kvh rows
  const size_t kvh = (size_t)(b * a.Hkv + g) * a.kv_rows;
  const auto qrs = make_rsrc((const __bf16*)a.q + (size_t)bh * a.q_rows * DQK,
                             (unsigned)((size_t)a.q_rows * DQK * 2));

  // ---- tile schedule -------------------------------------------------------------
  RingTiles ring;
  int ntiles;
  if (MODE == MODE_RING) {
    ring.init(a.q_part0 + part, a.P, a.Sp, BK, a.causal != 0, a.striped != 0, last_row - part * a.Sp);
    ntiles = ring.ntiles;
  } else {
    long long kmax = a.Sk;
    if (a.causal) kmax = min(kmax, last_pos - a.k_pos0 + 1);
    if (kmax <= 0) return;  // no key of this block is visible: state stays as it is
    ntiles = (int)((kmax + BK - 1) / BK);
  }
  // the same tiles in order, one step at a time (no divisions on the way)
  RingTiles::Cursor cursor;
  if (MODE == MODE_RING) cursor = ring.start();
  int walk_n = 0;
  auto walk_ref = [&]() __attribute__((always_inline)) -> TileRef {
    TileRef t;
    if (MODE == MODE_RING) {
      ring.at(cursor, t.row0, t.pos0, t.nvalid);
    } else {
      t.row0 = walk_n * BK;
      t.pos0 = a.k_pos0 + (long long)walk_n * BK;
      t.nvalid = min(BK, a.Sk - walk_n * BK);
    }
    return t;
  };
  auto walk_next = [&]() __attribute__((always_inline)) {
    if (MODE == MODE_RING)
      ring.advance(cursor);
    else
      ++walk_n;
  };
  // ---- direct HBM -> LDS tiles (unpadded, swizzled rows) ---------------------------
  // A 256-byte row holds 16 chunks of 16 bytes; chunk c of row r sits in slot
  // c ^ swz(r). swz is a bijection on 16 consecutive rows (conflict-free K reads of
  // one chunk across 16 rows) and, on the 4 rows x 2 chunk pairs that a half wave's
  // transposed V read touches, puts every pair on its own 8 banks.
  auto swz = [](int r) __attribute__((always_inline)) {
    const int x = r & 7;
    return ((((x & 3) << 1) | (x >> 2)) << 1) | ((r >> 3) & 1);
  };
  constexpr int ROWB = DQK * 2, ROWBV = DV * 2;
  constexpr bool SWZ = C::DMA || C::DMAW;
  constexpr int NI = SWZ ? BK * ROWBV / 1024 / NWS : 1;    // 1 KB V loads per wave per tile
  constexpr int NIK = C::DMAW ? BK * ROWB / 1024 / NWS : 1; // 1 KB K loads per wave per tile (384-byte rows)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // 384-byte K rows (D_qk = 192): the low three bits of chunk c of row r are XORed
  // with (r >> 1) & 7, which keeps c within its group of 8 chunks. Consecutive rows
  // start 32 banks apart, so the 16 rows of a 16-byte read of one chunk fall on 16
  // distinct 4-bank groups. A 1 KB load covers 2 2/3 rows, so each lane's global
  // offset is precomputed per load.
  auto kswz = [](int r) __attribute__((always_inline)) { return (r >> 1) & 7; };
  unsigned dgo[NI], dgok[NIK];
  if constexpr (SWZ) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = wave * (BK / NWS) + 4 * j + (lane >> 4);
      dgo[j] = (unsigned)(row * ROWBV + 16 * ((lane & 15) ^ swz(row)));
    }
  }
  if constexpr (C::DMAW) {
#pragma unroll
    for (int q = 0; q < NIK; ++q) {
      const int b = 1024 * (wave * NIK + q) + 16 * lane;
      const int row = b / ROWB, slot = (b - row * ROWB) / 16;
      dgok[q] = (unsigned)(row * ROWB + 16 * (slot ^ kswz(row)));
    }
  }
  const unsigned kv_bytes_last = (unsigned)((size_t)a.kv_rows * ROWBV - 16);
  const unsigned k_bytes_last = (unsigned)((size_t)a.kv_rows * ROWB - 16);
  const u32x4 kdesc = raw_desc((const __bf16*)a.k + kvh * DQK, (unsigned)((size_t)a.kv_rows * DQK * 2));
  const u32x4 vdesc = raw_desc((const __bf16*)a.v + kvh * DV, (unsigned)((size_t)a.kv_rows * DV * 2));
  // this stream's two buffers
  const unsigned k_lds = lds_addr(&ks[2 * stream][0]), v_lds = lds_addr(&vs[2 * stream][0]);
  // other head dims: the same direct loads into the padded rows, 1 KB piece by piece
  PaddedTileDma<BK, DQK * 2, C::KS * 2, NWS> kpad;
  PaddedTileDma<BK, DV * 2, C::VS * 2, NWS> vpad;
  if constexpr (!SWZ) {
    kpad.init(wave_u, lane);
    vpad.init(wave_u, lane);
  }
  auto dma_tile = [&](const TileRef& t, int buf) __attribute__((always_inline)) {
    if constexpr (C::DMAW) {
      const unsigned kbase = (unsigned)t.row0 * ROWB, vbase = (unsigned)t.row0 * ROWBV;
#pragma unroll
      for (int q = 0; q < NIK; ++q)
        lds_load16(k_lds + (unsigned)(buf * C::K_TILE * 2 + 1024 * (wave_u * NIK + q)), min(kbase + dgok[q], k_bytes_last),
                   kdesc);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        lds_load16(v_lds + (unsigned)(buf * C::V_TILE * 2 + (wave_u * (BK / NWS) + 4 * j) * ROWBV),
                   min(vbase + dgo[j], kv_bytes_last), vdesc);
    } else if constexpr (!C::DMA) {
      kpad.issue(wave_u, k_lds + (unsigned)(buf * C::K_TILE * 2), (unsigned)t.row0 * (DQK * 2),
                 (unsigned)((size_t)a.kv_rows * DQK * 2 - 16), kdesc);
      vpad.issue(wave_u, v_lds + (unsigned)(buf * C::V_TILE * 2), (unsigned)t.row0 * (DV * 2),
                 (unsigned)((size_t)a.kv_rows * DV * 2 - 16), vdesc);
    } else {
      const unsigned base = (unsigned)t.row0 * ROWB;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        // rows past the slab re-read its last chunk: finite values under the mask
        const unsigned off = min(base + dgo[j], kv_bytes_last);
        // K and V rows are both 256 bytes here, so one row offset serves both tiles
        const unsigned row_off = (unsigned)((wave_u * (BK / NWS) + 4 * j) * ROWB);
        lds_load16(k_lds + (unsigned)(buf * C::K_TILE * 2) + row_off, off, kdesc);
        lds_load16(v_lds + (unsigned)(buf * C::V_TILE * 2) + row_off, off, vdesc);
      }
    }
  };

  // ---- stationary Q fragments and running state --------------------------------
  const int wave_row0 = row_base + wave * NQ * 32;
  const long long wave_pos0 = pos_base + __builtin_amdgcn_readfirstlane(wave) * NQ * 32;   // wave-uniform
  bf16x8 qf[NQ][C::DS];
  float m[NQ], l[NQ];
  bool fresh[NQ];   // the row has no keys yet: its first visible tile sets m to the max
  f32x16 oacc[NQ][C::MT];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int row = wave_row0 + nq * 32 + l32;
    const bool valid = row < row_end;
#pragma unroll
    for (int s = 0; s < C::DS; ++s)
      qf[nq][s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (unsigned)(row * DQK + 16 * s + 8 * h) * 2u));
    m[nq] = 0.f;   // reference shift (exp2 domain)
    l[nq] = 0.f;
    fresh[nq] = true;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) oacc[nq][mt] = f32x16{};
    if (MODE == MODE_STEP && valid && stream == 0) {
      // running state (O normalised, LSE) is the online state with m = LSE, l = 1
      const size_t r = (size_t)bh * a.q_rows + row;
      const float lin = a.lse_acc[r];
      if (lin != kNegInf) {
        m[nq] = lin * kLog2e;
        l[nq] = h == 0 ? 1.f : 0.f;
        fresh[nq] = false;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = *(const f32x4*)(a.o_acc + r * DV + 32 * mt + 8 * g4 + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[nq][mt][4 * g4 + e] = x[e];
          }
      }
    }
  }

  // ---- one KV tile: S for all its keys, one online-softmax update, then PV --------
  const int gg = lane >> 4, L = lane & 15;
  // swizzled LDS byte addresses inside a tile: K chunk 2s+h of row l32, and the
  // transposed V read of row 8x + r4, column block mt
  unsigned kra[C::DMAW ? 8 : C::DS], vra[2][C::MT];
  if constexpr (C::DMA) {
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      kra[s] = k_lds + (unsigned)(l32 * ROWB + 16 * ((2 * s + h) ^ swz(l32)));
      asm volatile("" : "+v"(kra[s]));   // keep the lane base in a register: tile offsets stay immediates
    }
  }
  if constexpr (C::DMAW) {
    // chunk 2s + h = 8 (s / 4) + (2 (s % 4) + h): the XOR only touches the low three
    // bits, so four bases per buffer cover all twelve D steps
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kra[4 * b + u] = k_lds + (unsigned)(b * C::K_TILE * 2 + l32 * ROWB + 16 * ((2 * u + h) ^ kswz(l32)));
        asm volatile("" : "+v"(kra[4 * b + u]));
      }
  }
  if constexpr (SWZ) {
    const int r4 = 4 * (gg >> 1) + (L >> 2);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const int c = 4 * mt + 2 * (gg & 1) + ((L >> 1) & 1);
        vra[x][mt] = v_lds + (unsigned)((8 * x + r4) * ROWBV + 16 * (c ^ swz(8 * x + r4)) + 8 * (L & 1));
        asm volatile("" : "+v"(vra[x][mt]));
      }
  }
  auto kfrag = [&](int buf, int krow0, int s) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (C::DMA)
      return *(RA_LDS const bf16x8*)(uintptr_t)(kra[s] + (unsigned)(buf * C::K_TILE * 2 + krow0 * ROWB));
    else if constexpr (C::DMAW)
      return *(RA_LDS const bf16x8*)(uintptr_t)(kra[4 * buf + (s & 3)] + (unsigned)(128 * (s >> 2) + krow0 * ROWB));
    else
      return *(const bf16x8*)&ks[2 * stream + buf][(krow0 + l32) * C::KS + 16 * s + 8 * h];
  };
  auto compute_tile = [&](int buf, const TileRef& t, bool need_mask) __attribute__((always_inline)) {
    static_assert(NQ == 1, "one 32-row query block per wave");
    constexpr int NS = BK / 32;   // 32-key blocks of the S^T accumulator
    f32x16 sacc[NS];
    // D step outer, key block inner: each step issues NS independent MFMAs, and the
    // next step's NS K fragments are read from LDS while they run (the scheduling
    // barriers keep the compiler from trading that lead for registers)
    bf16x8 kc[NS], kn[NS];
#pragma unroll
    for (int kt = 0; kt < NS; ++kt) kc[kt] = kfrag(buf, kt * 32, 0);
#pragma unroll
    for (int kt = 0; kt < NS; ++kt) sacc[kt] = f32x16{};
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      if (s + 1 < C::DS) {
#pragma unroll
        for (int kt = 0; kt < NS; ++kt) kn[kt] = kfrag(buf, kt * 32, s + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < NS; ++kt) sacc[kt] = mfma32(kc[kt], qf[0][s], sacc[kt]);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < C::DS) {
#pragma unroll
        for (int kt = 0; kt < NS; ++kt) kc[kt] = kn[kt];
      }
    }
    if (need_mask) {
      // ragged tile or causal diagonal: keys past the last visible one become -inf.
      // lim = last visible key of block kt for this lane's query, minus the lane's
      // 4*h row offset, so each element compares a compile-time key offset
#pragma unroll
      for (int kt = 0; kt < NS; ++kt) {
        int lim = t.nvalid - 1 - kt * 32;
        if (a.causal) {
          const long long rel = wave_pos0 + l32 - (t.pos0 + kt * 32);
          lim = (int)min((long long)lim, max(rel, -1LL));
        }
        lim -= 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key_off = 8 * (i >> 2) + (i & 3);
          sacc[kt][i] = key_off <= lim ? sacc[kt][i] : kNegInf;
        }
      }
    }
    // the tile's row max of the raw scores (scale > 0)
    float mx = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < NS; ++kt)
#pragma unroll
      for (int i = (kt == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
    mx = row_max_halves(mx);
    // the shift moves to the tile max for rows whose scores lead it by more than
    // kLazyShift, and for rows seeing their first keys (so that a row's dominant
    // first key has P = 1 exactly, as with a running max). The branch is taken by
    // the whole wave; rows that keep their shift use sh = 0.
    const float lead = mx * a.scale_log2 - m[0];   // -inf for a row with nothing visible
    const bool move = lead > kLazyShift || (fresh[0] && mx != kNegInf);
    fresh[0] = fresh[0] && mx == kNegInf;
    if (__any(move)) {
      const float sh = move ? lead : 0.f;
      m[0] += sh;
      // A row that had keys before moves only by sh > kLazyShift, so its correction
      // 2^-sh is below one. A row seeing its first keys has l = 0 and a zero
      // accumulator, and its shift may move by any amount, also far downwards
      // (every score of the tile strongly negative), where 2^-sh would overflow
      // to +inf and 0 * inf would be NaN. Capping the exponent at 0 keeps the
      // correction finite for every row and changes nothing for the others.
      const float alpha = exp2_hw(fminf(-sh, 0.f));
      l[0] *= alpha;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) oacc[0][mt] *= alpha;
    }
    // P = exp2(scale * log2(e) * s - m), its row sum, and P^T in bf16 (round to
    // nearest even) straight from the accumulator registers
    bf16x8 pb[NS][2];
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < NS; ++kt) {
      f32x8 p0, p1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p0[i] = exp2_hw(fmaf(sacc[kt][i], a.scale_log2, -m[0]));
        p1[i] = exp2_hw(fmaf(sacc[kt][8 + i], a.scale_log2, -m[0]));
      }
      pb[kt][0] = to_bf16x8(p0);
      pb[kt][1] = to_bf16x8(p1);
#pragma unroll
      for (int i = 0; i < 8; ++i) rs += p0[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) rs += p1[i];
    }
    l[0] += rs;
    // O^T += V^T P^T, 16 keys per MFMA step. Step t2 of block kt holds, in lane
    // half h, keys 32*kt + 16*t2 + 4*h + {0..3} and 32*kt + 16*t2 + 8 + 4*h + {0..3}
    // (the accumulator rows of S^T); 16-lane group gg reads those keys for columns
    // 32*mt + 16*(gg%2) + 0..15 of the V tile, transposed.
    auto vread = [&](int it, bf16x4 (&f)[2][2]) __attribute__((always_inline)) {
      const int kt = it / C::MT, mt = it % C::MT;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          if constexpr (SWZ) {
            f[t2][x] = lds_read_tr16_at(vra[x][mt] + (unsigned)(buf * C::V_TILE * 2 + (kt * 32 + 16 * t2) * ROWBV));
          } else {
            const int dcol = 32 * mt + 16 * (gg & 1) + 4 * (L & 3);
            const int key = kt * 32 + 16 * t2 + 8 * x + 4 * (gg >> 1) + (L >> 2);
            f[t2][x] = lds_read_tr16(&vs[2 * stream + buf][key * C::VS + dcol]);
          }
        }
    };
    // the V^T fragments of step (kt, mt) + 1 are read while the products of (kt, mt)
    // run; the scheduling barriers keep that lead
    bf16x4 vc[2][2], vn[2][2];
    vread(0, vc);
#pragma unroll
    for (int it = 0; it < NS * C::MT; ++it) {
      const int kt = it / C::MT, mt = it % C::MT;
      if (it + 1 < NS * C::MT) vread(it + 1, vn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) oacc[0][mt] = mfma32(cat(vc[t2][0], vc[t2][1]), pb[kt][t2], oacc[0][mt]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int x = 0; x < 2; ++x) vc[t2][x] = vn[t2][x];
    }
  };

  // ---- pipelined tile loop -------------------------------------------------------
  const long long wave_pos1 = wave_pos0 + NQ * 32 - 1;
  auto tile_flags = [&](const TileRef& t, bool& skip, bool& need_mask) __attribute__((always_inline)) {
    skip = a.causal && t.pos0 > wave_pos1;
    need_mask = (t.nvalid < BK) || (a.causal && t.pos0 + BK - 1 > wave_pos0);
  };
  // Stream s takes tiles s, s + SPLIT, s + 2 SPLIT, ... of the schedule (SPLIT = 1:
  // every tile). Each stream's next tile streams into its other buffer (last read
  // before the previous barrier) while its current tile is computed; every step
  // ends with one barrier of the whole workgroup, so both streams run the same
  // number of steps (the second may have no tile in the last one). The loop is
  // unrolled by two so that every LDS address is a lane base plus an immediate.
  const int nsteps = (ntiles + SPLIT - 1) / SPLIT;
  TileRef t = walk_ref();
  if (SPLIT == 2 && stream == 1 && ntiles > 1) {
    walk_next();
    t = walk_ref();
  }
  if (SPLIT == 1 || stream < ntiles) dma_tile(t, 0);
  wait_vmem();
  __syncthreads();
  auto step = [&](int k, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int n = k * SPLIT + stream;   // this stream's tile
    bool skip, need_mask;
    tile_flags(t, skip, need_mask);
    TileRef tn = t;
    if (n + SPLIT < ntiles) {
#pragma unroll
      for (int sx = 0; sx < SPLIT; ++sx) walk_next();
      tn = walk_ref();
      dma_tile(tn, buf ^ 1);
    }
    if ((SPLIT == 1 || n < ntiles) && !skip) compute_tile(buf, t, need_mask);
    t = tn;
    wait_vmem();   // this wave's loads of its next tile have landed
    __syncthreads();
  };
  for (int k = 0; k < nsteps; k += 2) {
    step(k, std::integral_constant<int, 0>{});
    if (k + 1 < nsteps) step(k + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge of the two key streams (SPLIT = 2) ------------------------------------
  // Each stream holds the online state of the same rows over half of the keys.
  // Stream 1 hands its shift, exp-sum and accumulator to stream 0 through LDS (the
  // tiles are no longer read after the last barrier), which combines them: with
  // M the larger of the two shifts, both sides are scaled by 2^(shift - M) before
  // they are added (a side that saw no key contributes nothing).
  if constexpr (SPLIT == 2) {
    static_assert(NWS * C::MT * 4 * 64 * 16 <= sizeof(ks) && NWS * 64 * 2 * 4 <= sizeof(vs), "merge buffers");
    f32x4* xo = (f32x4*)&ks[0][0];     // [row group][4 MT][64 lanes] f32x4, conflict-free
    float* xm = (float*)&vs[0][0];     // [row group][64 lanes] shift, then exp-sum
    float* xl = xm + NWS * 64;
    if (stream == 1) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[0][mt][4 * g4 + e];
          xo[((wave * C::MT + mt) * 4 + g4) * 64 + lane] = x;
        }
      xm[wave * 64 + lane] = fresh[0] ? kNegInf : m[0];
      xl[wave * 64 + lane] = l[0];
    }
    __syncthreads();
    if (stream == 1) return;   // no barrier follows
    const float mine = fresh[0] ? kNegInf : m[0];
    const float other = xm[wave * 64 + lane];
    const float mm = fmaxf(mine, other);
    if (mm != kNegInf) {
      const float fa = mine == kNegInf ? 0.f : exp2_hw(mine - mm);
      const float fb = other == kNegInf ? 0.f : exp2_hw(other - mm);
      m[0] = mm;
      fresh[0] = false;
      l[0] = fa * l[0] + fb * xl[wave * 64 + lane];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 x = xo[((wave * C::MT + mt) * 4 + g4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[0][mt][4 * g4 + e] = fa * oacc[0][mt][4 * g4 + e] + fb * x[e];
        }
    }
  }

  // ---- epilogue ------------------------------------------------------------------
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const float lt = l[nq] + shfl_xor_f(l[nq], 32);
    const int row = wave_row0 + nq * 32 + l32;
    if (row < row_end) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? (m[nq] + log2_hw(lt)) * kLn2 : kNegInf;
      const size_t r = (size_t)bh * a.q_rows + row;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[nq][mt][4 * g4 + e] * inv;
          const int d = 32 * mt + 8 * g4 + 4 * h;
          if (MODE == MODE_RING)
            *(bf16x4*)((__bf16*)a.o + r * DV + d) = to_bf16x4(x);
          else
            *(f32x4*)(a.o_acc + r * DV + d) = x;
        }
      if (h == 0) {
        if (MODE == MODE_RING)
          a.lse[r] = lse;
        else
          a.lse_acc[r] = lse;
      }
    }
  }
}

// Workgroups of the launch for a given rows-per-workgroup.
static long long prefill_items(const PrefillArgs& a, int mode, int bq, int& n_qtiles) {
  const int rows_per_part = mode == MODE_RING ? a.Sp : a.q_rows;
  n_qtiles = (rows_per_part + bq - 1) / bq;
  return (long long)a.B * a.Hq * (mode == MODE_RING ? a.nq : 1) * n_qtiles;
}

template <int DQK, int DV, int MODE, int SPLIT>
static hipError_t launch_cfg(PrefillArgs a, hipStream_t st) {
  // 8 waves of 32 query rows: two waves per SIMD, so one wave's softmax (VALU)
  // overlaps the other's MFMAs, and each wave's working set fits in VGPRs.
  constexpr int NQ = 1, NW = 8;
  using C = PCfg<DQK, DV, NQ, NW, SPLIT>;
  const long long tiles = prefill_items(a, MODE, C::BQ, a.n_qtiles);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7ffffff0LL) return hipErrorInvalidValue;
  // whole rounds of the 8 XCDs (and, when blocks are dealt, of whole blocks)
  long long grid = 8 * ((tiles + 7) / 8);
  if ((a.B * a.Hkv) % 8 != 0) {
    const long long bs = (long long)kXcdTiles * (a.Hq / a.Hkv);
    grid = 8 * ((tiles + 8 * bs - 1) / (8 * bs)) * bs;
  }
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<DQK, DV, NQ, NW, MODE, SPLIT>), dim3((unsigned)grid),
                     dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

// One workgroup runs per CU (its LDS tiles fill most of the CU's 160 KB). A launch
// of fewer 256-row workgroups than two rounds of the chip's 256 CUs is short and
// bound by its heaviest workgroup, which under a causal mask walks up to twice the
// average key range; those launches split every workgroup's key range over two
// streams of waves (128 rows per workgroup), which halves that critical path.
constexpr long long kSplitBelow = 2 * 256;

template <int DQK, int DV, int MODE>
static hipError_t launch_one(PrefillArgs a, hipStream_t st) {
  int nqt;
  if (prefill_items(a, MODE, PCfg<DQK, DV, 1, 8, 1>::BQ, nqt) < kSplitBelow) return launch_cfg<DQK, DV, MODE, 2>(a, st);
  return launch_cfg<DQK, DV, MODE, 1>(a, st);
}

// Returns hipErrorInvalidValue when no kernel instance covers (dqk, dv).
hipError_t prefill_bf16(const PrefillArgs& a, int dqk, int dv, int step_mode, hipStream_t st) {
  if (dqk == 128 && dv == 128)
    return step_mode ? launch_one<128, 128, MODE_STEP>(a, st) : launch_one<128, 128, MODE_RING>(a, st);
  if (dqk == 64 && dv == 64)
    return step_mode ? launch_one<64, 64, MODE_STEP>(a, st) : launch_one<64, 64, MODE_RING>(a, st);
  if (dqk == 192 && dv == 128)
    return step_mode ? launch_one<192, 128, MODE_STEP>(a, st) : launch_one<192, 128, MODE_RING>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
