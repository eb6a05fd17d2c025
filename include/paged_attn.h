/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged-attention library
 * (libpaged_attn.so).
 *
 * The operations follow the pages' statement of the problem:
 *   - weft, "Shapes and symbols" and "Cache layouts": the per-layer paged cache
 *     view is [N, P, H_kv, D]; writes scatter through slot_mapping, reads gather
 *     through block_table; H_q / H_kv is the GQA group size G.
 *   - ember, "The core idea, in one picture": logical position p of a sequence
 *     lives at block block_table[p / P], offset p % P.
 *   - tiny-vllm-py, "KV Cache" (Mental Model, Design Choices, Mistakes I made):
 *     a query at position t attends to every cached token up to and including t;
 *     a new token's position is the cache length before its K/V is appended;
 *     prefill is causal and decode is unmasked.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, dense row-major, owned by the
 *     caller.  The library keeps no pointer after a call returns and allocates
 *     no memory; scratch space is a caller-provided workspace.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream).  None synchronises or reads device memory on the host.
 *   - Element type `dtype`: PA_DTYPE_F32 (float) or PA_DTYPE_BF16 (bfloat16).
 *     Arithmetic is fp32; outputs are written in the input dtype (bf16 rounded
 *     to nearest even).  Index arrays are int32.
 *   - Supported head_dim: 64 and 128.  Any block_size >= 1.  Any
 *     num_q_heads that is a multiple of num_kv_heads.
 *   - Scalars are validated before any HIP call; a zero-sized batch is a no-op
 *     that returns PA_OK.
 *   - Device metadata that is out of range (a slot outside [0, N*P), a block id
 *     outside [0, N), context_lens above max_blocks_per_seq * block_size) gives
 *     unspecified output values but never an out-of-bounds access: such slots
 *     are skipped, such tokens are masked, such lengths are clamped.
 *   - Return value: PA_OK (0) or a negative pa_status; pa_last_error() then
 *     holds a message for the calling thread.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PA_DTYPE_FP8_E4M3 (uint8 codes, see pa_reshape_and_cache_fp8)
 * is accepted by pa_copy_blocks only; the fp8 calls take it implicitly. */
typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1, PA_DTYPE_FP8_E4M3 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* null pointer, negative size, inconsistent shape  */
  PA_ERR_UNSUPPORTED = -2, /* well-formed but not provided (head_dim, dtype)    */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the size query */
  PA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed        */
} pa_status;

/* Library version (major * 10000 + minor * 100 + patch). */
int pa_version(void);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_slot_mapping -- slot of every new token (weft "Cache layouts"; ember
 * "The core idea").  Request b has T_b = cu_seqlens[b+1] - cu_seqlens[b] new
 * tokens and context_lens[b] cached tokens counting them, so its new token i sits
 * at position p = context_lens[b] - T_b + i and gets
 *     slot_mapping[cu_seqlens[b] + i] = block_table[b][p / P] * P + p % P,
 * the row index into the flattened [N * P] token rows of the pool.  Positions
 * outside [0, max_blocks_per_seq * P), negative block ids and slots beyond
 * 2^31 - 1 get slot -1; a block id at or past num_blocks gives a slot at or
 * past num_blocks * P.  pa_reshape_and_cache skips both, so such a token is
 * stored nowhere, as in pa_paged_decode_append.
 *   block_table  int32 [num_seqs, max_blocks_per_seq]
 *   cu_seqlens   int32 [num_seqs + 1], non-decreasing, cu_seqlens[0] = 0,
 *                cu_seqlens[num_seqs] = num_tokens
 *   context_lens int32 [num_seqs]
 *   slot_mapping int32 [num_tokens] (output)
 */
int pa_slot_mapping(const int32_t* block_table, const int32_t* cu_seqlens,
                    const int32_t* context_lens, int32_t* slot_mapping,
                    int32_t num_seqs, int64_t num_tokens, int32_t block_size,
                    int32_t max_blocks_per_seq, void* stream);

/*
 * pa_reshape_and_cache -- scatter new keys and values into the block pool
 * (weft "Cache layouts": write = scatter via slot_mapping; tiny-vllm-py
 * "Paged KV Cache", Mental Model: append into the tail block).  For every token
 * t with 0 <= slot_mapping[t] < num_blocks * block_size the [H_kv, D] row of k
 * (and of v) is copied bit for bit to row slot_mapping[t] of the pool viewed as
 * [N * P, H_kv, D].  Negative (padding) and out-of-range slots are skipped.
 * Slots must be distinct within one call (duplicates race).
 *   k, v               [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping       int32 [num_tokens]
 *   k_cache, v_cache   [num_blocks, block_size, num_kv_heads, head_dim], in place
 */
int pa_reshape_and_cache(const void* k, const void* v, const int32_t* slot_mapping,
                         void* k_cache, void* v_cache, int64_t num_tokens,
                         int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, void* stream);

/*
 * fp8 paged KV (ember, "Deliberately out of scope (for now)": paged KV
 * quantisation is a next step; the pages fix no format, so this library's
 * reading is): pools of uint8 OCP FP8 E4M3 codes (1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinities, largest magnitude 448), with
 * one fp32 scale per KV head for K and one for V.  Element x of KV head h is
 * stored as encode(x / scale[h]) -- the quotient correctly rounded to fp32,
 * then rounded to the nearest code with ties to even, magnitudes above 448
 * saturated to +-448 and NaN stored as 0x7F -- and read as decode(code) *
 * scale[h] (a NaN code reads as NaN).  Attention over an fp8 pool is
 * attention over those values.
 *
 * pa_reshape_and_cache_fp8 -- pa_reshape_and_cache into fp8 pools.
 *   k, v               [num_tokens, num_kv_heads, head_dim], dtype (F32 or BF16)
 *   k_cache, v_cache   uint8 [num_blocks, block_size, num_kv_heads, head_dim]
 *   k_scale, v_scale   float [num_kv_heads], device pointers, positive
 * head_dim must be a multiple of 16.  Slot rules as pa_reshape_and_cache.
 */
int pa_reshape_and_cache_fp8(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                             void* v_cache, const float* k_scale, const float* v_scale, int64_t num_tokens,
                             int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, void* stream);

/*
 * pa_paged_decode_append -- one decode step of a layer in one call: the step's
 * new token of each request is appended to the pools and attended to, exactly
 * as pa_reshape_and_cache (with the slots of positions context_lens[b] - 1)
 * followed by pa_paged_decode_attention, bit for bit (tiny-vllm-py "KV Cache":
 * the new token's K/V are stored first and the token sees itself; weft "Cache
 * layouts": the write is a scatter through the block table).
 *   k_new, v_new       [num_seqs, num_kv_heads, head_dim], dtype: the new token
 *                      of request b, stored at position context_lens[b] - 1
 *   k_cache, v_cache   written at those slots only (a block id outside
 *                      [0, num_blocks) is skipped, as the scatter skips such
 *                      slots; context_lens[b] == 0 or above max_blocks_per_seq
 *                      * block_size appends nothing)
 * Other arguments, the workspace and the errors are those of
 * pa_paged_decode_attention.  The pools must not hold the slot in more than
 * one request's table (a shared block is copied before it is appended to).
 */
int pa_paged_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* context_lens, float scale, void* out,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_paged_decode_attention_fp8 -- pa_paged_decode_attention over fp8 pools
 * (format and scales as above).  q and out are bfloat16; q's elements must lie
 * inside the fp16 range (the products run on fp16 matrix cores: the codes
 * widen exactly to fp16, and bf16 q converts exactly within that range).
 * Other arguments, the workspace and the errors are those of
 * pa_paged_decode_attention.
 */
int pa_paged_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, const int32_t* block_table, const int32_t* context_lens,
                                  float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * pa_paged_decode_append_fp8 -- pa_paged_decode_append over fp8 pools: equal,
 * bit for bit, to pa_reshape_and_cache_fp8 of the new rows (quantised with
 * k_scale / v_scale) followed by pa_paged_decode_attention_fp8.  k_new and
 * v_new are of type new_dtype (PA_DTYPE_F32 or PA_DTYPE_BF16); q and out are
 * bfloat16.  Errors: those of pa_paged_decode_append, and PA_ERR_UNSUPPORTED
 * for another new_dtype.
 */
int pa_paged_decode_append_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const float* k_scale, const float* v_scale, const int32_t* block_table,
                               const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_blocks_per_seq, int32_t new_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * pa_copy_blocks -- copy-on-write support for prefix sharing (tiny-vllm-py,
 * "Prefix Sharing": requests with a common prefix point their block tables at
 * the same physical blocks; a shared, partly filled block must be copied
 * before one request appends to it; ember, "Deliberately out of scope":
 * copy-on-write block tables).  For each pair, block dst of k_cache and of
 * v_cache becomes a bit-for-bit copy of block src.  Reads need nothing else:
 * attention through a table that shares blocks equals attention through one
 * that points at copies.
 *   k_cache, v_cache   [num_blocks, block_size, num_kv_heads, head_dim], in place
 *   block_mapping      int32 [num_pairs, 2]: (src, dst) per pair
 * Destinations must be distinct and must not be sources (the pairs run
 * concurrently); a pair with an entry outside [0, num_blocks) is skipped.
 * Same dtype and row-size rules as pa_reshape_and_cache.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int64_t num_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                   int32_t dtype, void* stream);

/*
 * pa_check_metadata -- checks device metadata against the rules the other
 * calls assume (they never read out of bounds when a rule is broken, but their
 * output is then unspecified).  Rules, as bits of result[0]:
 *   PA_CHECK_LENGTH        0 <= context_lens[b] <= max_blocks_per_seq * block_size
 *   PA_CHECK_BLOCK_ID      the first ceil(context_lens[b] / block_size) entries
 *                          of block_table row b lie in [0, num_blocks)
 *   PA_CHECK_CU_SEQLENS    cu_seqlens starts at 0, never decreases and ends at
 *                          num_tokens (only when cu_seqlens is given)
 *   PA_CHECK_CHUNK_LENGTH  cu_seqlens[b+1] - cu_seqlens[b] <= context_lens[b]
 *   PA_CHECK_SLOT          slot_mapping[t] < num_blocks * block_size (negative
 *                          slots are padding; only when slot_mapping is given)
 * result[1] counts the offending entries.  result is a device int32[2] that the
 * call overwrites; read it after the stream reaches the call.  cu_seqlens and
 * slot_mapping may be NULL.  Duplicate slots are not detected.
 */
#define PA_CHECK_LENGTH 1
#define PA_CHECK_BLOCK_ID 2
#define PA_CHECK_CU_SEQLENS 4
#define PA_CHECK_CHUNK_LENGTH 8
#define PA_CHECK_SLOT 16
int pa_check_metadata(const int32_t* block_table, const int32_t* context_lens, const int32_t* cu_seqlens,
                      const int32_t* slot_mapping, int32_t num_seqs, int64_t num_tokens, int64_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t* result, void* stream);

/* Bytes of workspace pa_paged_decode_attention needs for these shapes. */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq);

/*
 * pa_paged_decode_attention -- one query token per request attends, without a
 * mask, to the context_lens[b] tokens of its request, gathered through the block
 * table (tiny-vllm-py "KV Cache": the new token sees all earlier tokens and
 * itself; the scatter of this step's K/V happens before this call).  Query head
 * h reads KV head h / G, G = num_q_heads / num_kv_heads.
 *     out[b, h] = sum_j softmax_j(scale * q[b, h] . k_j) v_j,  j < context_lens[b]
 * context_lens[b] == 0 gives a zero row.
 *   q, out             [num_seqs, num_q_heads, head_dim] (out must not alias)
 *   k_cache, v_cache   [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_table        int32 [num_seqs, max_blocks_per_seq]; only the first
 *                      ceil(context_lens[b] / block_size) entries are read
 *   context_lens       int32 [num_seqs]
 *   workspace          device scratch of at least pa_decode_workspace_size()
 *                      bytes, not shared with a concurrently running call.
 *                      Its contents on entry do not matter (no clearing is
 *                      needed, also between calls or HIP graph replays); on
 *                      return it holds scratch values only.
 * The call enqueues two kernels (three for batches above 1024 requests, where
 * a separate kernel lists the work items).
 */
int pa_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens,
                              float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_paged_decode_attention_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc): pa_paged_decode_attention with the same arguments but no
 * workspace, giving the same result bit for bit.  Its workspace is a static
 * device array of PA_NOALLOC_SCRATCH_BYTES bytes inside the library, of which
 * each GPU the call runs on holds one copy until the process ends.  The call
 * allocates nothing.
 *   Batches whose pa_decode_workspace_size() exceeds PA_NOALLOC_SCRATCH_BYTES
 *   return PA_ERR_WORKSPACE before any HIP call (160 MiB holds, e.g., 256
 *   requests of up to 8192 tokens with 32 query heads of 128 dims).
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (other streams, concurrent graph replays) race and must not be
 *   made.  The array needs no clearing between calls.
 *   The first call on a device resolves the array's address there (with that
 *   device current) and keeps it; later calls reuse it.
 */
#define PA_NOALLOC_SCRATCH_BYTES (160u << 20)
int pa_paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                                      void* stream);

/*
 * pa_workspace_status -- reports whether a call that used this workspace left
 * work uncomputed.  The decode, decode-with-append and mixed calls hand out
 * their work items through queue counters that the first workgroup of each
 * launch resets; a wave that finds a counter not yet reset sleeps and tries
 * again, and after 2^20 sleeps gives that queue up, so that every wave
 * terminates.  The queue's remaining items are then not computed and the
 * output is wrong.  (The grid never exceeds the resident workgroups and the
 * first one resets the counters before its own claims, so this is not
 * expected to happen.)  Each give-up sets a bit of a status word in the
 * workspace header: 1 = a decode queue, 2 = a prefill queue of the mixed call.
 *   workspace  a workspace of pa_paged_decode_attention(_fp8),
 *              pa_paged_decode_append(_fp8) or pa_paged_mixed_attention(_fp8),
 *              or NULL for the static scratch of
 *              pa_paged_decode_attention_noalloc on the stream's device
 *   result     int32 device pointer; receives the bits set since the previous
 *              pa_workspace_status call on this workspace, and the word is
 *              cleared.  A new workspace holds arbitrary bits: its first status
 *              call only clears them (the static scratch starts at zero).
 * Runs asynchronously on stream, after the calls enqueued before it.
 * Setting the environment variable PA_TEST_QUEUE_GIVEUP=1 makes every queue
 * claim give up at once (for tests of this path).
 */
int pa_workspace_status(void* workspace, int32_t* result, void* stream);

/* Bytes of workspace pa_paged_prefill_attention needs for these shapes. */
size_t pa_prefill_workspace_size(int32_t num_seqs, int64_t total_q_tokens,
                                 int32_t num_q_heads, int32_t num_kv_heads);

/*
 * pa_paged_prefill_attention -- varlen and chunked prefill over the paged cache
 * (tiny-vllm-py "Mistakes I made": prefill is causal; ember "Deliberately out of
 * scope": chunked prefill; weft "Shapes and symbols": T_total packing).
 * k and v ARE the layer's paged pools, already holding this step's chunk
 * (written by pa_reshape_and_cache).  Request b's chunk has
 * T_b = cu_seqlens[b+1] - cu_seqlens[b] tokens; its row i sits at absolute
 * position L_b - T_b + i (L_b = context_lens[b]) and attends causally to keys
 * 0 .. L_b - T_b + i.  Requests with T_b > L_b produce unspecified rows.
 *   q, out        [total_q_tokens, num_q_heads, head_dim], packed by request
 *   k, v          [num_blocks, block_size, num_kv_heads, head_dim]
 *   cu_seqlens    int32 [num_seqs + 1]
 *   block_table   int32 [num_seqs, max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 *   workspace     at least pa_prefill_workspace_size() bytes
 * dtype must be PA_DTYPE_BF16 (bf16 MFMA); fp32 returns PA_ERR_UNSUPPORTED, as
 * does max_blocks_per_seq above 16384 (a request's block ids are staged on
 * chip).  scale must be positive and finite (PA_ERR_INVALID otherwise).
 */
int pa_paged_prefill_attention(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens, const int32_t* block_table,
                               const int32_t* context_lens, float scale, void* out,
                               int32_t num_seqs, int64_t total_q_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_paged_prefill_attention_fp8 -- pa_paged_prefill_attention over fp8 pools
 * (uint8 E4M3 codes with per-KV-head scales, as for
 * pa_paged_decode_attention_fp8; q and out bfloat16, q inside the fp16 range).
 * Other arguments, the workspace and the errors are those of
 * pa_paged_prefill_attention.
 */
int pa_paged_prefill_attention_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                                   const float* v_scale, const int32_t* cu_seqlens, const int32_t* block_table,
                                   const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                   int64_t total_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                   int32_t max_blocks_per_seq, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Bytes of workspace pa_paged_mixed_attention needs for these shapes. */
size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq);

/*
 * pa_paged_mixed_attention -- one step's ragged mix of decode requests and
 * prefill chunks in a single persistent launch (tiny-vllm-py "KV Cache": a
 * step may mix prefill and decode, which wants ragged batches and a kernel
 * that takes both; ember "Deliberately out of scope": a prefill/decode mix
 * per step).  It computes exactly what pa_paged_prefill_attention computes on
 * the same arguments: request b's chunk of T_b = cu_seqlens[b+1] -
 * cu_seqlens[b] tokens, row i at absolute position L_b - T_b + i, attending
 * causally to keys 0 .. L_b - T_b + i; a chunk of one token is a decode step
 * over all L_b keys.  One-token chunks are computed as the decode call's
 * split-context partitions (merged by a second, small kernel), longer chunks
 * as the prefill call's items; requests with T_b > L_b (or T_b = 0) leave
 * their rows untouched.
 *   q, out        [total_q_tokens, num_q_heads, head_dim], packed by request
 *   k, v          [num_blocks, block_size, num_kv_heads, head_dim]
 *   cu_seqlens    int32 [num_seqs + 1]
 *   block_table   int32 [num_seqs, max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 *   workspace     at least pa_mixed_workspace_size() bytes, not shared with a
 *                 concurrently running call; its contents on entry do not
 *                 matter (as for pa_paged_decode_attention)
 * Restrictions and errors are those of pa_paged_prefill_attention, plus:
 * num_seqs above 1024 returns PA_ERR_UNSUPPORTED (the work lists are derived
 * on chip), as do batches whose work lists exceed 2^24 - 8192 items.
 */
int pa_paged_mixed_attention(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             const int32_t* block_table, const int32_t* context_lens, float scale, void* out,
                             int32_t num_seqs, int64_t total_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_paged_mixed_attention_fp8 -- pa_paged_mixed_attention over fp8 pools
 * (uint8 E4M3 codes with per-KV-head scales, as for
 * pa_paged_decode_attention_fp8; q and out bfloat16, q inside the fp16 range).
 * Other arguments, the workspace and the errors are those of
 * pa_paged_mixed_attention.
 */
int pa_paged_mixed_attention_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                                 const float* v_scale, const int32_t* cu_seqlens, const int32_t* block_table,
                                 const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                 int64_t total_q_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * pa_set_timing_events -- measurement hook.  While both events are non-NULL
 * (hipEvent_t handles), each attention call on this thread records `start`
 * just before and `stop` just after its main kernel (the decode partition
 * kernel, the prefill kernel or the mixed kernel), on the call's stream, so the caller can time
 * that kernel alone with hipEventElapsedTime.  Pass NULL, NULL to turn it off.
 */
int pa_set_timing_events(void* start_event, void* stop_event);

/*
 * pa_hbm_read -- measurement aid, not a step of the attention path: streams
 * `bytes` (a multiple of 16) from `src` (device, 16-byte aligned) with
 * nontemporal 16-byte loads over `num_workgroups` workgroups of 256 threads
 * and stores nothing but, with negligible probability, one word to `sink`
 * (device, one uint32).  Its rate is the practical HBM read ceiling that the
 * decode kernel's gathers (which also read from HBM only) are compared with.
 * Errors: PA_ERR_INVALID for a negative or unaligned size, num_workgroups
 * outside [1, 2^20], a null pointer or an unaligned src.  bytes == 0 is a
 * no-op.
 */
int pa_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
