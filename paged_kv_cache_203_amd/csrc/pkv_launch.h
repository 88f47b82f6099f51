// Internal launch interface between the C-ABI layer (pkv_api.hip) and the kernels
// (pkv_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_check.h"

namespace pkv {

struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* context_lens;
  void* out;             // single pass: [B, Hq, D] in the element type
  float* partial_out;    // split: [B, Hq, max_partitions, D]
  float* partial_lse;    // split: [B, Hq, max_partitions]
  float scale_log2;      // scale * log2(e): scores are kept in the base-2 domain
  int32_t batch, hq, hkv, group;
  int32_t num_pages, max_pages, page_shift, capacity;   // capacity = max_pages * page_size
  int32_t partition_tokens, max_partitions;
  int32_t part_begin;    // split: first partition launched (the ones before are written elsewhere)
  int32_t heads_per_wg;  // KV heads per workgroup (divides hkv and the wave count)
  int32_t tok_stride;    // bytes between consecutive slots of a page (Hkv * D * elem)
  int64_t page_stride;   // bytes per page (page_size * tok_stride)
};

// Balanced decode step: `a` carries the attention arguments (heads_per_wg set; the partition
// fields are unused).  Workspace (laid out by step_workspace): per-(sequence, head group)
// arrival counters ws_count (generation-tagged words, see pkv_arrival.h; zero before the first
// call, and every completed call leaves them at zero), piece partials ws_out
// [(groups + B) * Hq * D] and ws_lse [(groups + B) * Hq].
struct StepParams {
  DecodeParams a;
  const void* k_new;     // null: no append
  const void* v_new;
  void* k_pool_w;        // the pools, writable (the appended rows)
  void* v_pool_w;
  float* ws_out;
  float* ws_lse;
  uint64_t* ws_count;
  uint32_t generation;   // this call's generation (pkv_arrival.h), never 0
  void* out;
  float* lse_out;        // may be null
  int32_t groups;        // token-range groups per head group
  int32_t append;        // 1: append k_new/v_new at context_lens[b], attend over +1
  // 1: the waves that share a KV head (heads_per_wg < 8) each stream all of its tiles for their
  // own ceil(group / waves per head) query heads (the launch's padded group is that count);
  // 0: they take turns on its tiles, each for the whole group.
  int32_t qsplit;
  // Rotary embedding (with the append only): the new key is written rotated and q is rotated
  // in registers, both at position context_lens[b]; rope_cos / rope_sin [rope_rows, D/2].
  const float* rope_cos; // null: no rotation
  const float* rope_sin;
  int32_t rope_rows;
  // Multi-query decode (q_tokens = T > 1, no append, no rotation): the step runs over T x Hq
  // heads (a.hq = T x Hq, a.group = T x the GQA group); head kvh * a.group + c is query token
  // c / (a.group / T) of query head kvh * (a.group / T) + c % (a.group / T), attending to tokens
  // t <= L - T + (its query token); q, out, lse_out are [batch, T, Hq].  0 or 1: the decode step.
  int32_t q_tokens;
};

struct MergeParams {
  const float* partial_out;
  const float* partial_lse;
  const int32_t* context_lens;
  void* out;
  float* lse_out;        // may be null
  int32_t batch, hq, partition_tokens, max_partitions, capacity;
  // q_tokens = T > 1: rows are (sequence, query token j) pairs, batch * T of them, and row
  // (b, j) covers L_b - T + 1 + j tokens (multi-query decode); 0 or 1: one query per sequence.
  int32_t q_tokens;
};

// Shared-prefix partitions: every sequence's tokens [0, prefix_tokens) sit in the pages
// prefix_pages[0 .. prefix_tokens / page_size).  Partitions [0, prefix_tokens / partition_tokens)
// of the split-KV partials are written (bf16 and fp16 only).
struct PrefixParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* prefix_pages;
  const int32_t* context_lens;
  float* partial_out;    // [B, Hq, max_partitions, D]
  float* partial_lse;    // [B, Hq, max_partitions]
  float scale_log2;
  int32_t batch, hq, hkv, group;
  int32_t num_pages, page_shift, capacity;
  int32_t prefix_tokens, partition_tokens, max_partitions;
  int32_t tok_stride;
  int64_t page_stride;
  // Multi-query decode (q_tokens = T > 0): q [B, T, Hq, D], partials [B, T, Hq, max_partitions, D];
  // every sequence's pages come from its page_table row (max_pages entries); prefix_* unused.
  const int32_t* page_table;
  int32_t max_pages, q_tokens;
};

struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* page_table;
  const int32_t* context_lens;
  int32_t batch, num_pages, max_pages, page_shift, capacity;
  int32_t row_bytes;     // Hkv * D * elem: one slot of one pool
  int64_t page_stride;
};

// Fused rotary embedding + append: q -> q_out rotated, k_new rotated into the K pool, v_new into
// the V pool, at position context_lens[b]; the rotary cache is rope_cos / rope_sin
// [rope_rows, D/2] float32.
struct RopeParams {
  AppendParams a;
  const void* q;
  void* q_out;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_rows, hq, hkv;
};

// Whole-page copies in both pools (copy-on-write of shared pages): pairs [n][2] = (src, dst).
struct CopyPagesParams {
  void* k_pool;
  void* v_pool;
  const int32_t* pairs;
  int32_t n, num_pages;
  int64_t page_bytes;
};

struct ValidateParams {
  const int32_t* page_table;
  const int32_t* context_lens;
  int32_t* device_status;
  int32_t batch, num_pages, max_pages, page_size, extra_tokens, check_append_unique;
};

// Each returns hipSuccess or the launch error.  `dtype` is a pkv_dtype; `group_pad` is the
// padded GQA group (4, 8 or 16).
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int group_pad,
                         bool partial, hipStream_t stream);
// Waves per decode workgroup; heads_per_wg must divide it.
int decode_waves();
hipError_t launch_step(const StepParams& p, int dtype, int head_dim, int group_pad,
                       hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t stream);
// Multi-query decode (p.q_tokens > 0) on the matrix cores; bf16 and fp16 only.
hipError_t launch_prefix(const PrefixParams& p, int dtype, int head_dim, hipStream_t stream);
// Shared-prefix decode, both kinds of partition in one launch: `d` as for launch_decode's
// partial mode (suffix partitions from d.part_begin), `pp` as for launch_prefix (q_tokens = 0).
// bf16 and fp16 only.
hipError_t launch_cascade(const DecodeParams& d, const PrefixParams& pp, int dtype, int head_dim,
                          int group_pad, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_rope_append(const RopeParams& p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_validate(const ValidateParams& p, hipStream_t stream);
hipError_t launch_copy_pages(const CopyPagesParams& p, hipStream_t stream);
// Zero `bytes` (a multiple of 16) of device memory at `dst` (16-byte aligned) with a kernel.
hipError_t launch_zero(void* dst, uint64_t bytes, hipStream_t stream);
// Plain read stream of `bytes` (a multiple of 16) from `src` over `workgroups` workgroups; each
// folds what it read into *sink (XOR).
hipError_t launch_read_stream(const void* src, uint64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream);

}  // namespace pkv
