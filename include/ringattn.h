/*
 * ringattn.h — C ABI of the MI355X (gfx950) ring-ordered blockwise exact attention
 * library (libringattn.so).
 *
 * What it computes. For a query block and a sequence of KV blocks, exact
 * O = softmax(scale * Q K^T) V and the per-row log-sum-exp of the scaled scores,
 * built one KV block at a time: each block updates a per-row running maximum and
 * exp-sum, rescales the output accumulator and merges the block's contribution,
 * so the result equals one-shot attention.
 *   [RING] page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条超长序列",
 *          §"KV 在 Ring 中如何流动" (ring order) and §"最容易被忽略的细节：不同 Block 的
 *          Attention 结果不能直接相加" (running max / sum / rescale / merge).
 *   [IMPL] page "LLM长文本推理Ring Attention环形注意力机制实现与优化",
 *          §"Ring Attention实现代码与通信重叠" (lse state, initial out = 0, lse = -inf,
 *          the rescale weights of the old output and the block output).
 *   [CH]   page "长上下文的第一性挑战", §挑战 1 eq. lc-ch-attention (definition),
 *          §KV 是 Decode 阶段的隐性瓶颈 (decode reads the whole KV cache once).
 *   [CPEV] page "上下文并行 (CP) 收益评估实验设计", §名词定义 (pass-KV / pass-Q) and
 *          §Decode (partial attention on every KV shard, then a reduction).
 *
 * Conventions shared by every call.
 *   - Tensors are dense, contiguous, row-major "BHSD": batch, head, sequence,
 *     head-dim (innermost). LSE tensors are [B, H, S] fp32 (natural log, scale
 *     included). Pointers marked "device" are HIP device memory owned by the
 *     caller; the library never allocates, frees or synchronises.
 *   - dtype: RA_F32 (fp32 in, fp32 arithmetic) or RA_BF16 (bf16 in, fp32
 *     accumulation, softmax probabilities rounded to bf16 for the PV product,
 *     outputs rounded to nearest-even bf16).
 *   - Causal visibility uses global token positions: a key is visible to a query
 *     iff key_pos <= query_pos.
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *   - A query with no visible key gets O = 0 and LSE = -inf.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream. Work is
 *     enqueued asynchronously on it; results are valid once the stream has been
 *     synchronised.
 *   - Return value: RA_OK, or an error code with a message in ra_last_error().
 *     No call throws. Arguments are validated before anything is enqueued, so an
 *     error return has enqueued no work.
 *   - The library keeps no state between calls apart from the per-thread error
 *     message; calls are reentrant.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 5

typedef enum {
  RA_OK = 0,
  RA_EINVAL = 1,        /* null pointer, bad size, inconsistent shapes, misalignment */
  RA_EUNSUPPORTED = 2,  /* valid request with no kernel instance for it (dtype, head dims, slab size) */
  RA_EHIP = 3           /* the HIP runtime reported an error at launch */
} ra_status;

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* ABI version of the loaded library (RA_ABI_VERSION of the headers it was built with). */
int ra_abi_version(void);

/* Message for the last non-OK return on the calling thread ("" if none). The pointer
 * stays valid until the next library call on the same thread. */
const char* ra_last_error(void);

/* Host only, no GPU. Ring visiting order of query partition i in a ring of P
 * partitions ([RING] §"KV 在 Ring 中如何流动"): at step s the partition works on KV
 * block kv_block[s] = (i - s) mod P. kind[s] is 0 = skip (causal and the block lies
 * wholly after partition i), 1 = diagonal (causal, own block, masked elementwise),
 * 2 = full. kv_block and kind are host arrays of at least P ints.
 * Returns P, or -RA_EINVAL on bad arguments. */
int ra_ring_schedule(int P, int i, int causal, int* kv_block, int* kind);

/* Ring prefill for nq consecutive query partitions, all in one launch ([RING]
 * §"KV 在 Ring 中如何流动": every device keeps its query block while the KV blocks
 * travel round the ring, so partition i meets block (i - s) mod P at step s, and
 * under a causal mask blocks holding only future tokens contribute nothing).
 * The sequence has P * Sp tokens cut into P contiguous partitions of Sp tokens.
 *   q   device [B, Hq,  nq*Sp, Dqk]  queries of partitions q_part0 .. q_part0+nq-1
 *   k   device [B, Hkv, P*Sp,  Dqk]  all P KV blocks (block j = tokens j*Sp ..)
 *   v   device [B, Hkv, P*Sp,  Dv ]
 *   o   device [B, Hq,  nq*Sp, Dv ]  output, same dtype as q
 *   lse device [B, Hq,  nq*Sp] fp32  output
 * Each query partition i visits KV blocks in the order of ra_ring_schedule(P, i,
 * causal), skipping "skip" blocks and masking the diagonal one; the running state
 * stays in registers across the blocks.
 * Supported head dims: RA_BF16 (Dqk, Dv) in {(64,64), (128,128), (192,128)};
 * RA_F32 Dqk, Dv in {64, 128}. scale must be finite and > 0.
 * Errors: RA_EINVAL for null pointers, non-positive sizes, Hq % Hkv != 0,
 * q_part0 + nq > P, pointers not 16-byte aligned; RA_EUNSUPPORTED for other head
 * dims or a per-(batch, head) slab of q, k, v or o of 2^31 bytes or more. */
int ra_ring_attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sp, int P, int q_part0, int nq, int Dqk, int Dv,
                     float scale, int causal, void* stream);

/* Striped layout ([IMPL] §长文本场景下的性能表现与调优: the striped variant deals
 * token positions to the devices round-robin so that, under a causal mask, every
 * device has visible keys in every ring step): partition p holds global tokens
 * p, p + P, p + 2P, ..., in that order. Key c of block j is visible to local query
 * row r of partition i iff c*P + j <= r*P + i. Fills kv_block[s] as
 * ra_ring_schedule and kind[s] = 1 (masked triangle) for every step when causal,
 * 2 otherwise; no step is skipped. Returns P, or -RA_EINVAL on bad arguments. */
int ra_ring_schedule_striped(int P, int i, int causal, int* kv_block, int* kind);

/* Ring prefill as ra_ring_attn_fwd, for the striped layout: row r of partition p
 * in q, k, v, o and lse is global token r*P + p. Visits the blocks in the order of
 * ra_ring_schedule_striped; under a causal mask each query tile reads every block
 * up to its own last local row. Without a causal mask the result equals
 * ra_ring_attn_fwd's. Arguments, head-dim support and errors as ra_ring_attn_fwd. */
int ra_ring_attn_fwd_striped(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Sp, int P, int q_part0, int nq, int Dqk, int Dv,
                             float scale, int causal, void* stream);

/* One ring step: merge one KV block into a running fp32 state ([IMPL] §Ring
 * Attention实现代码与通信重叠; [RING] §最容易被忽略的细节).
 *   q       device [B, Hq,  Sq, Dqk]  queries at global positions q_pos0 .. q_pos0+Sq-1
 *   k_blk   device [B, Hkv, Sk, Dqk]  keys at global positions k_pos0 .. k_pos0+Sk-1
 *   v_blk   device [B, Hkv, Sk, Dv ]
 *   o_acc   device [B, Hq,  Sq, Dv ] fp32, normalised running output (in/out)
 *   lse_acc device [B, Hq,  Sq] fp32, running log-sum-exp (in/out)
 * Start from o_acc = 0, lse_acc = -inf. After the call the state equals the merge
 * of the old state with exact attention over this block. A block with no visible
 * key for any query leaves the state untouched. Head-dim support and errors as
 * ra_ring_attn_fwd. o_acc/lse_acc must not overlap q, k_blk or v_blk. */
int ra_block_attn_step(int dtype, const void* q, long long q_pos0, int Sq,
                       const void* k_blk, const void* v_blk, long long k_pos0, int Sk,
                       int B, int Hq, int Hkv, int Dqk, int Dv, float scale, int causal,
                       float* o_acc, float* lse_acc, void* stream);

/* Two-way merge of normalised partial results over disjoint key sets, per row
 * ([IMPL] §"Ring Attention实现代码与通信重叠": the new lse of the union and the two
 * weights that rescale the old output and the block output; [RING]
 * §"最容易被忽略的细节": per-block softmax results cannot simply be added):
 * L = log(e^{La} + e^{Lb}); O = e^{La-L} O_a + e^{Lb-L} O_b. A side with -inf
 * LSE contributes nothing; two empty sides give O = 0, L = -inf.
 *   o_a, o_b, o_out  device [rows, Dv] fp32;  lse_a, lse_b, lse_out device [rows] fp32.
 * o_out/lse_out may alias o_a/lse_a (or o_b/lse_b) exactly; other overlaps are
 * undefined. Errors: RA_EINVAL for null pointers, rows < 0, Dv <= 0, Dv % 4 != 0,
 * pointers not 16-byte aligned. rows == 0 is a no-op. */
int ra_lse_merge(long long rows, int Dv, const float* o_a, const float* lse_a,
                 const float* o_b, const float* lse_b, float* o_out, float* lse_out, void* stream);

/* n-way reduction of partials, the pass-Q reduce ([CPEV] §Decode).
 *   o_parts   device [rows, n, Dv] fp32 normalised partial outputs
 *   lse_parts device [rows, n] fp32
 *   o_out     device [rows, Dv] in out_dtype (RA_F32 or RA_BF16)
 *   lse_out   device [rows] fp32
 * Errors: RA_EINVAL for null pointers, rows < 0, n <= 0, Dv <= 0, Dv % 4 != 0,
 * pointers not 16-byte aligned. rows == 0 is a no-op. */
int ra_lse_merge_n(int out_dtype, long long rows, int n, int Dv, const float* o_parts,
                   const float* lse_parts, void* o_out, float* lse_out, void* stream);

/* Split-KV decode: one new query token per sequence attends to its whole KV cache
 * (no mask: every cached key precedes it). The cache is cut into n_splits
 * contiguous chunks of L / n_splits keys; each chunk yields a partial (O_p, LSE_p),
 * then an LSE-weighted reduction gives the result ([CPEV] §名词定义 pass-Q;
 * [CH] §KV 是 Decode 阶段的隐性瓶颈).
 *   q        device [B, Hq, Dqk]
 *   k_cache  device [B, Hkv, L, Dqk]
 *   v_cache  device [B, Hkv, L, Dv]
 *   o_part   device [B, Hq, n_splits, Dv] fp32  output (partials)
 *   lse_part device [B, Hq, n_splits] fp32      output
 *   o        device [B, Hq, Dv] dtype of q       output
 *   lse      device [B, Hq] fp32                 output
 * Supported: RA_BF16 with Dqk == Dv in {64, 128} and Hq / Hkv <= 16 (the query
 * heads of one KV head share one matrix-core tile); anything else returns
 * RA_EUNSUPPORTED. Errors: RA_EINVAL for null pointers, non-positive sizes,
 * Hq % Hkv != 0, L % n_splits != 0, pointers (the partials and lse included) not
 * 16-byte aligned. */
int ra_splitkv_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                      int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                      float* o_part, float* lse_part, void* o, float* lse, void* stream);

/* The partial half of ra_splitkv_decode: only o_part / lse_part, no reduction.
 * This is what each KV shard computes before the partials are exchanged and
 * reduced with ra_lse_merge_n ([CPEV] §Decode). Arguments, support and errors as
 * ra_splitkv_decode without o / lse. */
int ra_splitkv_partial(int dtype, const void* q, const void* k_cache, const void* v_cache,
                       int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                       float* o_part, float* lse_part, void* stream);

/* Split-KV decode over an FP8 KV cache: one byte per cached value ([CH] §挑战 2
 * KV-size equation, b = 1 for FP8), so the cache scan that bounds decode
 * ([CH] §KV 是 Decode 阶段的隐性瓶颈) reads half the bytes of bf16.
 *   q        device [B, Hq, Dqk] bf16
 *   k_cache  device [B, Hkv, L, Dqk] fp8 e4m3 (OCP: 1 sign, 4 exponent bits with
 *            bias 7, 3 mantissa bits, no infinities, 0x7f / 0xff are NaN); the
 *            key used is k_scale times the stored value
 *   v_cache  device [B, Hkv, L, Dv] fp8 e4m3; the value used is v_scale times it
 *   o_part, lse_part, o (bf16), lse: as ra_splitkv_decode.
 * The stored values are widened exactly to bf16 for the products; k_scale
 * multiplies the scores (with scale) and v_scale the normalised outputs.
 * Supported: Dqk == Dv in {64, 128}, Hq/Hkv <= 16. Errors as ra_splitkv_decode,
 * plus RA_EINVAL for k_scale or v_scale not finite and > 0. */
int ra_splitkv_decode_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                          int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                          float* o_part, float* lse_part, void* o, float* lse, void* stream);

/* The partial half of ra_splitkv_decode_fp8 (no reduction), as ra_splitkv_partial. */
int ra_splitkv_partial_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                           int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                           float* o_part, float* lse_part, void* stream);

/* ra_splitkv_decode for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc):
 * the same partials and reduction, with the partials kept in a scratch array that
 * the library holds on each GPU (16 MiB per device, held until the process ends)
 * instead of caller buffers. Allocates nothing; the caller passes inputs and
 * outputs only.
 *   q, k_cache, v_cache, o, lse: as ra_splitkv_decode; supported shapes as there.
 * The partials [B, Hq, n_splits, Dv] fp32 and their LSEs must fit the scratch:
 * B * Hq * n_splits * (Dv + 1) * 4 bytes (plus alignment) <= 16 MiB, else RA_EINVAL
 * with the sizes in the message. The first call on a device looks the scratch up
 * with that device current: call it with the stream's device current. Every call
 * on one GPU shares that GPU's scratch, so calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results; calls ordered on one
 * stream are safe. Each call overwrites the partials completely, so nothing of an
 * earlier call leaks into a later one. Errors as ra_splitkv_decode, and RA_EHIP if
 * the scratch lookup fails. */
int ra_splitkv_decode_noalloc(int dtype, const void* q, const void* k_cache, const void* v_cache,
                              int B, int Hq, int Hkv, int L, int Dqk, int Dv, int n_splits, float scale,
                              void* o, float* lse, void* stream);

/* Backward pass. The pages run ring attention on training samples and name the
 * backward pass's data dependencies among what a ring must get right ([RING]
 * opening example; §什么时候值得引入 Context Parallelism); the gradients are those
 * of the attention definition ([CH] §挑战 1), with P = exp(scale q k - LSE) from
 * the forward's saved row LSE.
 *
 * delta[r] = sum_d dout[r, d] * o[r, d] in fp32, for `rows` rows of Dv values
 * (o: the forward output, dout: its incoming gradient; device, [rows, Dv], both
 * RA_BF16 or both RA_F32 as `dtype` says).
 * Errors: RA_EINVAL for null pointers or pointers (delta included) not 16-byte
 * aligned, rows < 0, Dv not a positive multiple of 8, a dtype other than RA_F32
 * or RA_BF16. */
int ra_attn_bwd_preprocess(int dtype, const void* o, const void* dout, long long rows, int Dv, float* delta,
                           void* stream);

/* One backward ring step: adds one (query block, KV block) pair's gradient
 * contributions to fp32 accumulators (which the caller zero-initialises):
 *   dv_acc += P^T dout,  dS = P o (dout V^T - delta),
 *   dq_acc += scale dS K, dk_acc += scale dS^T Q   (dk/dv summed over each KV
 *   head's query heads),  P = exp(scale Q K^T - lse) on the visible keys.
 *   q, dout  device [B, Hq,  Sq, Dqk / Dv] in dtype, queries at global positions q_pos0 ..
 *   lse, delta device [B, Hq, Sq] fp32: the queries' full-row LSE (forward output)
 *            and delta (ra_attn_bwd_preprocess); a row with LSE = -inf adds nothing
 *   k_blk, v_blk device [B, Hkv, Sk, Dqk / Dv] in dtype, keys at global positions k_pos0 ..
 *   dq_acc [B, Hq, Sq, Dqk], dk_acc [B, Hkv, Sk, Dqk], dv_acc [B, Hkv, Sk, Dv] fp32 (in/out)
 * A ring backward is this step for every (query block, KV block) pair, in any
 * order, with dk_acc / dv_acc travelling with their block. Two launches (dK/dV,
 * then dQ) on the stream. Supported: RA_BF16 with (Dqk, Dv) in {(64,64),
 * (128,128), (192,128)} (matrix cores; P and dS rounded to bf16 for the products)
 * and RA_F32 with Dqk, Dv in {64, 128} (fp32 matrix cores, fp32 throughout). Errors as
 * ra_block_attn_step. The accumulators must not overlap the inputs or each other. */
int ra_block_attn_bwd_step(int dtype, const void* q, const void* dout, const float* lse, const float* delta,
                           long long q_pos0, int Sq, const void* k_blk, const void* v_blk, long long k_pos0, int Sk,
                           int B, int Hq, int Hkv, int Dqk, int Dv, float scale, int causal, float* dq_acc,
                           float* dk_acc, float* dv_acc, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RINGATTN_H */
