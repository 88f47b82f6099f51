/*
 * pkv.h — C ABI of libpkv: single-token grouped-query decode attention over a paged KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation.  Each sequence b of a decode batch has one new query token q[b] (Hq heads of
 * head_dim D) and a context of L_b earlier tokens whose key and value rows live in fixed-size
 * pages of one shared pool.  Logical token t of sequence b is slot t % page_size of physical page
 * page_table[b][t / page_size].  Query head h attends with KV head h / (Hq / Hkv) (grouped-query
 * attention), and the result is softmax(scale * q K^T) V over the L_b tokens.
 *   - CacheIR page, "Compiler Example": decode lowers grouped_query_attention to one
 *     paged_attention_decode(q, k, v) call that receives the new token's k and v.
 *   - CacheIR page, "Current Capabilities" / "Boundaries": paged KV metadata over persistent
 *     shared page-backed KV pools, page-table decode attention with GQA mapping, a batched
 *     paged-attention ABI and a reduced (split-then-reduce) paged-attention decode.
 *   - TorchInferno page, "Custom Kernels": paged_decode_attention and
 *     batched_paged_decode_attention (one page table per request); "Runtime Scaffolds":
 *     runtime.paged holds page-table-shaped KV allocation; "OpenAI-Compatible Serving": separate
 *     KV-append, grouped decode and streaming (blockwise) decode kernels.
 *   - Sequences that share a prefix name the same physical pages in their tables (TorchInferno
 *     page, "Design Coverage": shared prefix-page reuse).
 *
 * Layouts (all row-major, contiguous, element type = pkv_shape.dtype unless stated):
 *   q            [batch, num_q_heads, head_dim]
 *   k_pool       [num_pages, page_size, num_kv_heads, head_dim]   (v_pool the same)
 *   page_table   int32 [batch, max_pages_per_seq]
 *   context_lens int32 [batch]
 *   out          [batch, num_q_heads, head_dim]          (same dtype as q)
 *   partial_out  float32 [batch, num_q_heads, max_partitions, head_dim]
 *   partial_lse  float32 [batch, num_q_heads, max_partitions]  (natural-log log-sum-exp)
 *   k_new, v_new [batch, num_kv_heads, head_dim]
 *
 * Ownership and ordering.  Every pointer argument (except `shape`, which is host memory read
 * during the call) is device memory owned by the caller.  The library allocates nothing, keeps
 * no pointer after returning, and only enqueues work on `stream` (a hipStream_t; NULL is the
 * null stream) without synchronising, except pkv_validate_metadata, which documents its own
 * behaviour.  The caller keeps buffers alive and unmodified until the enqueued work completes.
 * Device metadata is never modified.
 *
 * Errors.  Every call checks its arguments on the host before enqueuing anything and returns
 *   PKV_OK (0), PKV_EINVAL (-1, a bad argument), PKV_EUNSUPPORTED (-2, valid but not built:
 *   dtype, head_dim, page_size, group size), PKV_ELAUNCH (-3, the HIP launch failed) or
 *   PKV_EWORKSPACE (-4, a caller buffer too small).
 * On a non-zero return nothing was enqueued (PKV_ELAUNCH aside) and pkv_last_error() returns a
 * message for the calling thread.  There is no fallback path.
 *
 * Supported: dtype f32 / bf16 / f16; head_dim 64 or 128; page_size a power of two from 16 to
 * 256; num_q_heads a multiple of num_kv_heads with group size G = Hq / Hkv at most 16.
 *
 * Device-side metadata preconditions (page ids of live entries in [0, num_pages),
 * context_lens[b] <= max_pages_per_seq * page_size) cannot be read on the host without a sync;
 * pkv_validate_metadata checks them.  The kernels never read or write outside the pools when
 * they are violated: a row whose live page id is out of range, or whose length exceeds the
 * table's capacity, gets NaN outputs (attention) or is skipped (append).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_EINVAL (-1)
#define PKV_EUNSUPPORTED (-2)
#define PKV_ELAUNCH (-3)
#define PKV_EWORKSPACE (-4)

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_F16 = 2 } pkv_dtype;

/* Sizes shared by every call.  Element type `dtype` (a pkv_dtype) applies to q, the pools,
 * k_new, v_new and out. */
typedef struct {
  int32_t batch;              /* B >= 0 (0: nothing to do)                          */
  int32_t num_q_heads;        /* Hq > 0, a multiple of num_kv_heads                 */
  int32_t num_kv_heads;       /* Hkv > 0                                            */
  int32_t head_dim;           /* D: 64 or 128                                       */
  int32_t page_size;          /* PS: power of two, 16..256                          */
  int32_t num_pages;          /* NP > 0: pages in each pool                         */
  int32_t max_pages_per_seq;  /* MP > 0: page_table row length                      */
  int32_t dtype;              /* pkv_dtype                                          */
} pkv_shape;

/* Decode attention, one pass per (sequence, KV head).
 *
 * out[b, h, :] = sum_t softmax_t(scale * q[b,h] . K_b[t, h/G]) V_b[t, h/G, :] for t < L_b,
 * where K_b/V_b are the rows reached through page_table[b] and L_b = context_lens[b].
 * Accumulation is float32; out is rounded to the element type (round-to-nearest-even).
 * context_lens[b] <= 0 gives out[b] = 0.  Table entries past ceil(L_b / PS) and slots at or past
 * L_b in the last page are never read.  `scale` must be finite (usually 1/sqrt(D)).
 * `out` must not overlap q or the pools.
 * Follows the CacheIR page, "Compiler Example": in the decode-specialised graph, grouped-query
 * attention over the cached keys and values becomes one paged_attention_decode(q, k, v) call per
 * step; "Current Capabilities" names the multi-batch page-table form with the GQA head mapping.
 * The batched form with one page table per request is the TorchInferno page's
 * batched_paged_decode_attention ("Custom Kernels"). */
int pkv_paged_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* page_table, const int32_t* context_lens,
                               float scale, void* out, const pkv_shape* shape, void* stream);

/* Split-KV (flash-decoding) partial attention.
 *
 * Partition p of sequence b covers logical tokens [p*P, min((p+1)*P, L_b)) with
 * P = partition_tokens (a multiple of page_size).  For every p < ceil(L_b / P) it writes the
 * normalised partial output partial_out[b, h, p, :] (float32) and its log-sum-exp
 * partial_lse[b, h, p] = ln sum_t exp(scale * q . k_t) over the partition.  Partitions at or past
 * ceil(L_b / P) are not written.  max_partitions (the third dimension of both buffers) must be at
 * least ceil(max_pages_per_seq * page_size / P), else PKV_EWORKSPACE.  Results depend only on
 * the sequence's own tokens and P, never on the batch around it.  This follows the "reduced
 * paged-attention decode" of the CacheIR page ("Current Capabilities") and the blockwise
 * streaming decode of the TorchInferno page ("OpenAI-Compatible Serving"); the split itself is
 * the flash-decoding form. */
int pkv_paged_decode_attention_partial(const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* page_table, const int32_t* context_lens,
                                       float scale, int32_t partition_tokens,
                                       float* partial_out, float* partial_lse,
                                       int32_t max_partitions, const pkv_shape* shape,
                                       void* stream);

/* Log-sum-exp merge of the partitions written by pkv_paged_decode_attention_partial.
 *
 * With n_b = ceil(L_b / P) partitions, M = max_p lse_p and w_p = exp(lse_p - M):
 *   out[b, h, :] = sum_p w_p partial_out[b, h, p, :] / sum_p w_p   (rounded to the element type)
 *   lse_out[b, h] = M + ln sum_p w_p                               (float32; lse_out may be NULL)
 * Rows with L_b <= 0 get out = 0 and lse_out = -inf.  `out` must not overlap the partials.
 * This is the reduce half of the CacheIR page's reduced (split, then reduced) paged-attention
 * decode ("Current Capabilities", native backend row); the pages give no formula for the
 * reduction, and the one above is the exact combination of softmax partials by their
 * log-sum-exps. */
int pkv_lse_merge(const float* partial_out, const float* partial_lse,
                  const int32_t* context_lens, int32_t partition_tokens, int32_t max_partitions,
                  void* out, float* lse_out, const pkv_shape* shape, void* stream);

/* Shared-prefix (cascade) decode: paged decode attention for a batch whose sequences all begin
 * with the same prefix_tokens tokens, stored once in the pool.
 *
 * Token t < prefix_tokens of every sequence is slot t % PS of page prefix_pages[t / PS]
 * (prefix_pages holds prefix_tokens / PS page ids; the page tables' first prefix_tokens / PS
 * entries are not read); tokens t >= prefix_tokens are found through page_table as usual.  The
 * result is that of pkv_paged_decode_attention over L_b = context_lens[b] tokens (rows with
 * L_b < prefix_tokens attend to their first L_b prefix tokens only), computed as two launches
 * on `stream`:
 *   1. one grid holding both kinds of partition, which share no data and run side by side:
 *      - the prefix partitions p < prefix_tokens / P (P = partition_tokens): for each KV head,
 *        the query rows of all sequences (B x G rows) attend to the prefix as one dense product
 *        on the matrix cores, so each prefix page is read once per 128 query rows, not once per
 *        sequence;
 *      - the remaining partitions, as pkv_paged_decode_attention_partial computes them;
 *   2. the merge of all ceil(L_b / P) partitions, as pkv_lse_merge.
 * partial_out / partial_lse are the caller's workspace in the split layout (their contents after
 * the call are the partitions' partials); out and lse_out (may be NULL) are as for
 * pkv_lse_merge.  This follows the shared prefix-page reuse of the TorchInferno page ("Design
 * Coverage") and the Infinity docs' direction of sharing one block store across related
 * requests ("Short shared prefix qualification"); the split into prefix and suffix partitions
 * merged by log-sum-exp is the cascade form of the split-KV decode.
 *
 * Requirements: dtype bf16 or f16 (else PKV_EUNSUPPORTED); partition_tokens a multiple of 64 and
 * of page_size, with partition_tokens / page_size <= 512; prefix_tokens a multiple of
 * partition_tokens in [0, max_pages_per_seq * page_size]; max_partitions as for the split call.
 * Prefix page ids outside [0, num_pages) give NaN outputs for the rows that reach them.  The
 * partials' bits depend only on the sequence's own tokens and P; the prefix partials are not
 * bitwise those of the split call (a different summation order), but agree to rounding. */
int pkv_paged_decode_cascade(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* prefix_pages, int32_t prefix_tokens,
                             const int32_t* page_table, const int32_t* context_lens, float scale,
                             int32_t partition_tokens, float* partial_out, float* partial_lse,
                             int32_t max_partitions, void* out, float* lse_out,
                             const pkv_shape* shape, void* stream);

/* Paged KV append: the new token's key and value rows of every sequence are copied, bit for
 * bit, into the pools at logical position L_b = context_lens[b] (the pre-append length), i.e.
 * slot L_b % PS of page page_table[b][L_b / PS].  Rows with context_lens[b] < 0 are padding and
 * write nothing.  No other byte of the pools changes; re-running it writes the same bytes.
 * Attention afterwards is called with context_lens + 1.  Destinations must be distinct across
 * rows and must not be a page another row reads (check with pkv_validate_metadata); padding rows
 * never write.  (CacheIR page, "Compiler Example": the decode op receives the new k and v;
 * TorchInferno page, "OpenAI-Compatible Serving": the KV-append kernel.) */
int pkv_paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* page_table, const int32_t* context_lens,
                        const pkv_shape* shape, void* stream);

/* Multi-query paged decode: T = num_query_tokens new tokens per sequence (speculative or
 * suffix decode), attending causally.
 *
 * q and out are [batch, T, num_q_heads, head_dim].  context_lens[b] = L_b counts every token of
 * the sequence, the T new ones included (their K/V rows are already in the pages).  Query j
 * (0-based) sits at position L_b - T + j and attends to tokens 0 .. L_b - T + j through
 * page_table as usual, so each query is the decode of one token over its own prefix; queries
 * with no tokens (L_b - T + 1 + j <= 0) and padding rows get out = 0, lse = -inf.
 * Two launches on `stream`: for every (sequence, KV head, partition of P = partition_tokens
 * tokens), the G x T query rows attend to the partition's tokens as one dense product on the
 * matrix cores (the K and V of the partition are read once for all T queries; the same kernel
 * as the shared-prefix path's prefix partitions), writing partials to partial_out / partial_lse
 * ([batch, T, num_q_heads, max_partitions, (head_dim)], float32); then the log-sum-exp merge of
 * each query's ceil((L_b - T + 1 + j) / P) partitions into out and lse_out ([batch, T,
 * num_q_heads], float32, may be NULL).  The pages tile decode attention over up to 32 query rows
 * of suffix tokens after a cached context (Infinity docs, "Short shared prefix qualification");
 * the causal rule is that of decoder self-attention.
 *
 * Requirements: dtype bf16 or f16 (else PKV_EUNSUPPORTED); partition_tokens a multiple of 64 and
 * of page_size with partition_tokens / page_size <= 512; max_partitions >=
 * ceil(max_pages_per_seq * page_size / partition_tokens).  A row's bits depend only on its own
 * sequence, its query index and P. */
int pkv_paged_decode_multi_query(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* page_table, const int32_t* context_lens,
                                 int32_t num_query_tokens, float scale, int32_t partition_tokens,
                                 float* partial_out, float* partial_lse, int32_t max_partitions,
                                 void* out, float* lse_out, const pkv_shape* shape,
                                 void* stream);

/* Multi-query paged decode through the balanced decode step: the same result as
 * pkv_paged_decode_multi_query (T = num_query_tokens new tokens per sequence, q and out
 * [batch, T, num_q_heads, head_dim], lse_out [batch, T, num_q_heads] float32 or NULL,
 * context_lens[b] = L_b counting the T new tokens, whose K/V rows are already in the pages;
 * query j attends to tokens 0 .. L_b - T + j; queries with no tokens and padding rows get
 * out = 0, lse = -inf; rows longer than the page table can address get NaN), in one launch.
 * The T x G query rows of a KV head are the step's query columns: the batch's tiles are split
 * evenly over the GPU as in pkv_paged_decode_step, each tile is read once for all T queries, and
 * each column stops at its own query's position.  The pages tile decode attention over the
 * suffix tokens of a cached context (Infinity docs, "Short shared prefix qualification").
 * workspace: caller-owned device memory of pkv_multi_query_step_workspace_bytes(shape, T) bytes,
 * zero-filled once before the first call and then left as each call leaves it (as for
 * pkv_paged_decode_step; calls that overlap on one workspace race).
 * Requirements: dtype bf16 or f16 (else PKV_EUNSUPPORTED), T >= 1, T x (num_q_heads /
 * num_kv_heads) <= 128, T x num_q_heads <= 1024,
 * batch <= 4096.  A row's bits depend on the batch (as for the step); pkv_paged_decode_multi_query
 * gives bits that depend only on the row. */
int pkv_paged_decode_multi_query_step(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* page_table, const int32_t* context_lens,
                                      int32_t num_query_tokens, float scale, void* workspace,
                                      size_t workspace_bytes, void* out, float* lse_out,
                                      const pkv_shape* shape, void* stream);

/* Workspace bytes of pkv_paged_decode_multi_query_step for this shape and num_query_tokens on
 * the current device; 0 for an invalid shape or num_query_tokens < 1. */
size_t pkv_multi_query_step_workspace_bytes(const pkv_shape* shape, int32_t num_query_tokens);

/* Fused rotary embedding + paged KV append for the decode step's new token.
 *
 * For every row with L = context_lens[b] >= 0 (the new token's position), in one launch:
 *   q_out[b, h, :] = RoPE(q[b, h, :], L) for every query head h;
 *   the K pool slot L % PS of page page_table[b][L / PS] = RoPE(k_new[b], L), bit for bit;
 *   the same slot of the V pool = v_new[b], bit for bit.
 * RoPE is the rotate-half form: pair i < D/2 of a head is (x[i], x[i + D/2]), turned to
 * (x[i] c - x[i + D/2] s, x[i + D/2] c + x[i] s) with c = rope_cos[L][i], s = rope_sin[L][i]
 * (the caller's rotary cache, float32 [rope_positions, D/2], 16-byte aligned), computed in
 * float32 with each product and sum rounded to nearest even, then rounded to the element type.
 * The pages name this step (CacheIR page, "Compiler Example": rope(q, k) ahead of the decode
 * attention, fused_rmsnorm_qkv_rope ahead of paged_attention_decode; TorchInferno page,
 * "OpenAI-Compatible Serving": a decode rotary-append kernel) but not its formula; the
 * rotate-half form is that of the Llama/Mistral/Qwen decoders they target.
 * Padding rows (L < 0) copy q to q_out and write nothing.  Rows with L >= rope_positions or
 * L >= max_pages_per_seq * page_size get NaN in q_out and write nothing; a row whose page id is
 * out of range writes nothing.  q_out must not overlap any input.  Attention afterwards uses
 * q_out and context_lens + 1. */
int pkv_rope_kv_append(const void* q, const void* k_new, const void* v_new, void* k_pool,
                       void* v_pool, const int32_t* page_table, const int32_t* context_lens,
                       const float* rope_cos, const float* rope_sin, int32_t rope_positions,
                       void* q_out, const pkv_shape* shape, void* stream);

/* One whole decode step in one call, with the work split evenly over the GPU.
 *
 * With k_new and v_new non-NULL, every sequence's new K and V rows are first written into the
 * pools at position context_lens[b] (exactly as pkv_paged_kv_append), and attention then covers
 * context_lens[b] + 1 tokens.  With both NULL, the pools are only read and attention covers
 * context_lens[b] tokens.  out / lse_out are as for pkv_lse_merge (lse_out may be NULL); rows
 * with no tokens get out = 0, lse = -inf.
 *
 * The batch's tiles of 16 tokens are cut into equal contiguous ranges, one per workgroup and as
 * many workgroups as the GPU holds at once, so every compute unit gets the same share whatever
 * the mix of lengths; a range can hold pieces of several sequences, and the pieces of a sequence
 * are combined with the log-sum-exp rule (the flash-decoding split; CacheIR page, "Current
 * Capabilities": persistent multi-batch page-table decode).  Results agree with
 * pkv_paged_decode_attention to rounding and are deterministic for a given batch, but unlike the
 * fixed-partition calls their last bits can depend on the other sequences (the split points do).
 *
 * It is one launch: the workgroup that finishes the last piece of a sequence merges it, found
 * through per-sequence arrival counters kept in the workspace.
 *
 * workspace: caller-owned device memory of at least pkv_decode_step_workspace_bytes(shape)
 * bytes (queried on the same device), 16-byte aligned, zero-filled before its first use.  The
 * counters sit at its start, sized for the largest batch.  Each is tagged with the generation of
 * the call that last counted into it (every call of the step in a process takes a new, larger
 * generation on the host), so a count that an unfinished earlier call left behind is discarded
 * by the next call rather than merged; every completed call also leaves its counters at zero.
 * One workspace therefore serves later calls without clearing as long as num_kv_heads stays the
 * same (any batch up to the one it was sized for); zero it again before using it for another
 * head count.  A call captured in a graph keeps its generation for every replay, which the zeros
 * a completed replay leaves make safe.  Calls that share a workspace must not run concurrently.
 * Supports batch <= 4096 and num_q_heads <= 1024 (else PKV_EUNSUPPORTED). */
int pkv_paged_decode_step(const void* q, const void* k_new, const void* v_new, void* k_pool,
                          void* v_pool, const int32_t* page_table, const int32_t* context_lens,
                          float scale, void* workspace, size_t workspace_bytes, void* out,
                          float* lse_out, const pkv_shape* shape, void* stream);

/* pkv_paged_decode_step for callers that cannot allocate or hand over a workspace (code being
 * captured into a graph, tight serving loops, harnesses that forbid allocation): the same kernel,
 * its workspace taken from a static device array of the library (64 MiB, held on every GPU the
 * library runs on until the process ends) instead of a caller buffer.  Arguments, results and
 * bits are those of pkv_paged_decode_step with the same inputs.  The call allocates nothing; on
 * its first use on a device it looks up the array's device address and clears it with one kernel
 * on `stream`.  Shapes whose step workspace (pkv_decode_step_workspace_bytes) exceeds 64 MiB are
 * rejected with PKV_EWORKSPACE.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be serialised by the caller. */
int pkv_paged_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                  void* k_pool, void* v_pool, const int32_t* page_table,
                                  const int32_t* context_lens, float scale, void* out,
                                  float* lse_out, const pkv_shape* shape, void* stream);

/* The decode step with the rotary embedding fused in: as pkv_paged_decode_step with an append,
 * except that the new key is written rotated, and the query rotated, both at position
 * context_lens[b], exactly as pkv_rope_kv_append computes them (same float32 steps, same
 * rounding); attention then covers context_lens[b] + 1 tokens.  One launch does the rotation,
 * the append and the attention.  rope_cos, rope_sin, k_new and v_new must be non-NULL.  A row
 * whose position has no row in the rotary cache (context_lens[b] >= rope_positions) writes a NaN
 * key, so its output is NaN. */
int pkv_paged_decode_step_rope(const void* q, const void* k_new, const void* v_new, void* k_pool,
                               void* v_pool, const int32_t* page_table,
                               const int32_t* context_lens, const float* rope_cos,
                               const float* rope_sin, int32_t rope_positions, float scale,
                               void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                               const pkv_shape* shape, void* stream);

/* Workspace bytes pkv_paged_decode_step needs on the current device (0 on a bad shape or when
 * no device is available). */
size_t pkv_decode_step_workspace_bytes(const pkv_shape* shape);

/* Device-side check of the metadata preconditions.  Rows with L = context_lens[b] +
 * extra_tokens > 0 are live and use n = ceil(L / PS) table entries.  Writes one int32 status
 * word to device_status (stream-ordered; read it after the stream completes):
 *   bit 0 (1): a live table entry outside [0, num_pages)
 *   bit 1 (2): n > max_pages_per_seq (the length exceeds the table's capacity)
 *   bit 2 (4): with check_append_unique != 0, a row's append page (entry context_lens[b] / PS)
 *              is also a live entry of another row.
 * The host-side checks of every call cover what the host can see; this call covers the
 * device-resident metadata.  It follows the CacheIR page, "Boundaries" (paged KV-cache reference
 * behaviour and shared page allocator accounting among the implemented, tested boundaries) and
 * the Infinity docs, "Current execution limits", where every boundary and retained length is
 * checked before GPU work and destination rows must be unique and in range. */
int pkv_validate_metadata(const int32_t* page_table, const int32_t* context_lens,
                          int32_t extra_tokens, int32_t check_append_unique,
                          int32_t* device_status, const pkv_shape* shape, void* stream);

/* Whole-page copies in both pools, for copy-on-write: pairs is device int32 [n_pairs][2] of
 * (source page, destination page); every byte of each source page of k_pool and of v_pool is
 * copied to the destination page.  Pairs with a page outside [0, num_pages), or a page onto
 * itself, are skipped.  Destinations must be distinct and must not be sources of other pairs. */
int pkv_copy_pages(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                   const pkv_shape* shape, void* stream);

/* Host page allocator: which physical pages of the pools each sequence uses, with sharing.
 *
 * Host memory and host logic only (no device work, no stream).  Pages carry a reference count:
 * one per sequence that lists the page, one if the prefix cache holds it; a page whose count
 * reaches zero is free again, and the lowest free id is always taken first, so the ids handed
 * out depend only on the sequence of calls.  A sequence is a page list plus a token count; its
 * table row (pkv_pages_seq_table) and length are what the attention calls take as page_table
 * and context_lens.  This follows the shared page allocator accounting across forked request
 * sessions (CacheIR page, "Current Capabilities"), page-table-shaped KV allocation and a radix
 * prefix tree with prefix-cache lookup (TorchInferno page, "Runtime Scaffolds": runtime.paged,
 * runtime.prefix, runtime.prefix_cache).  Every call returns a PKV_* code; messages come from
 * pkv_pages_last_error().  One allocator must not be used from two threads at once. */
typedef struct pkv_page_allocator pkv_page_allocator;

/* A pool of num_pages pages of page_size tokens; NULL on bad arguments. */
pkv_page_allocator* pkv_pages_create(int32_t num_pages, int32_t page_size);
void pkv_pages_destroy(pkv_page_allocator* a);
int32_t pkv_pages_free_count(const pkv_page_allocator* a);
/* A page's reference count (-1 for a bad page id). */
int32_t pkv_pages_refcount(const pkv_page_allocator* a, int32_t page);
/* An empty sequence. */
int pkv_pages_seq_create(pkv_page_allocator* a, int32_t* seq_out);
/* A new sequence sharing every page of src, with src's length (a forked request). */
int pkv_pages_seq_fork(pkv_page_allocator* a, int32_t src, int32_t* seq_out);
/* Drop the sequence's references; its id may be reused. */
int pkv_pages_seq_release(pkv_page_allocator* a, int32_t seq);
/* Grow the sequence by n_tokens (their slots are [length, length + n_tokens), to be written by
 * an append).  If the last page is partly filled and shared, it is first replaced by a fresh page
 * and (old, fresh) is written to copies_out (room for max_copies pairs; *n_copies = 1): the
 * caller copies that page on the device (pkv_copy_pages) before appending.  New pages are taken
 * for the rest.  Without enough free pages nothing changes and PKV_EWORKSPACE is returned. */
int pkv_pages_seq_reserve(pkv_page_allocator* a, int32_t seq, int32_t n_tokens,
                          int32_t* copies_out, int32_t max_copies, int32_t* n_copies);
int pkv_pages_seq_length(const pkv_page_allocator* a, int32_t seq, int32_t* len_out);
/* The sequence's page-table row: its page ids, then -1 up to max_pages (PKV_EWORKSPACE if it has
 * more pages); *n_pages = its page count. */
int pkv_pages_seq_table(const pkv_page_allocator* a, int32_t seq, int32_t* row,
                        int32_t max_pages, int32_t* n_pages);
/* Register the sequence's first n_tokens (token ids) in the prefix cache, page by page: each
 * full page becomes a node (parent node, its page_size token ids) holding a reference to the
 * page, unless an equal node exists. */
int pkv_pages_prefix_insert(pkv_page_allocator* a, int32_t seq, const int32_t* tokens,
                            int32_t n_tokens);
/* A new sequence starting on the pages of the longest cached prefix of tokens (whole pages,
 * token ids compared exactly); *matched_tokens = its length. */
int pkv_pages_seq_create_with_prefix(pkv_page_allocator* a, const int32_t* tokens,
                                     int32_t n_tokens, int32_t* seq_out,
                                     int32_t* matched_tokens);
/* Evict up to max_pages cache nodes: least recently used leaves whose page only the cache holds. */
int pkv_pages_prefix_evict(pkv_page_allocator* a, int32_t max_pages, int32_t* evicted);
const char* pkv_pages_last_error(void);

/* Bytes of partial_out plus partial_lse for `max_partitions` partitions (0 on a bad shape). */
size_t pkv_partial_workspace_bytes(const pkv_shape* shape, int32_t max_partitions);

/* Plain read stream, for measurement: every byte of src[0, bytes) is read once with 16-byte
 * loads spread over the whole device (the direct-to-LDS loads the decode kernels stream K rows
 * with), and one 32-bit word per workgroup of what was read is folded by XOR into *sink (a device
 * uint32, not cleared here), so that no read is dead.  Its rate is the read bandwidth this device actually reaches, the
 * ceiling the decode calls' algorithmic bytes per second are reported against beside the
 * published HBM peak (the CacheIR page, "Latest local validation", reports a bandwidth
 * calibration beside its kernel timings).  src and bytes must be multiples of 16
 * (PKV_EINVAL otherwise). */
int pkv_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Message describing the calling thread's last non-zero return ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
