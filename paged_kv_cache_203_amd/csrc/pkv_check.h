// Host-side argument checks for the libpkv entry points.  Pure C++ (no HIP), so the checks can
// be built and unit-tested with any host compiler.  Each function returns a PKV_* code and, on
// failure, a message in `msg`.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/pkv.h"

namespace pkv {

// Element size in bytes of a pkv_dtype (0 if unknown).
int elem_bytes(int32_t dtype);

// Sizes every call shares: positive heads, Hq % Hkv == 0, supported D / PS / G / dtype.
// max_group: the largest num_q_heads / num_kv_heads accepted (16 for the attention calls; the
// multi-query step checks its T x Hq heads against its own limit).
int check_shape(const pkv_shape* s, std::string& msg, int max_group = 16);

// Byte extent of each tensor for a checked shape.
struct Extents {
  uint64_t q, pool, out, new_rows, table, lens;
};
Extents extents(const pkv_shape& s);

// Range overlap of [a, a+na) and [b, b+nb).
bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb);

int check_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                 const int32_t* context_lens, float scale, const void* out, const pkv_shape* s,
                 std::string& msg);

// Smallest max_partitions that covers every length the page table can address.
int32_t partitions_needed(const pkv_shape& s, int32_t partition_tokens);

int check_partial(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                  const int32_t* context_lens, float scale, int32_t partition_tokens,
                  const float* partial_out, const float* partial_lse, int32_t max_partitions,
                  const pkv_shape* s, std::string& msg);

int check_merge(const float* partial_out, const float* partial_lse, const int32_t* context_lens,
                int32_t partition_tokens, int32_t max_partitions, const void* out,
                const float* lse_out, const pkv_shape* s, std::string& msg);

int check_append(const void* k_new, const void* v_new, const void* k_pool, const void* v_pool,
                 const int32_t* page_table, const int32_t* context_lens, const pkv_shape* s,
                 std::string& msg);

// The rotary cache of the fused step: non-NULL, 16-byte aligned, rope_positions > 0, and no
// overlap with the step's outputs or workspace.
int check_rope_tables(const void* k_new, const float* rope_cos, const float* rope_sin,
                      int32_t rope_positions, const void* out, const float* lse_out,
                      const void* workspace, size_t workspace_bytes, const pkv_shape* s,
                      std::string& msg);

int check_rope_append(const void* q, const void* k_new, const void* v_new, const void* k_pool,
                      const void* v_pool, const int32_t* page_table, const int32_t* context_lens,
                      const float* rope_cos, const float* rope_sin, int32_t rope_positions,
                      const void* q_out, const pkv_shape* s, std::string& msg);

// Largest batch the balanced decode step supports (its tile prefix lives in LDS), and most query
// heads (keeps a sequence's piece partials within 32-bit buffer offsets).
constexpr int kMaxStepBatch = 4096;
constexpr int kMaxStepHeads = 1024;

// Shared-prefix decode: most prefix page ids one partition may span (they are staged in LDS), and
// the token block the partition length must be a multiple of.
constexpr int kMaxPrefixPageIds = 512;
constexpr int kPrefixBlock = 64;

int check_cascade(const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* prefix_pages, int32_t prefix_tokens, const int32_t* page_table,
                  const int32_t* context_lens, float scale, int32_t partition_tokens,
                  const float* partial_out, const float* partial_lse, int32_t max_partitions,
                  const void* out, const float* lse_out, const pkv_shape* s, std::string& msg);

int check_multi_query(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* page_table, const int32_t* context_lens, int32_t q_tokens,
                      float scale, int32_t partition_tokens, const float* partial_out,
                      const float* partial_lse, int32_t max_partitions, const void* out,
                      const float* lse_out, const pkv_shape* s, std::string& msg);

// Workspace layout of the balanced decode step for `groups` workgroup ranges (all offsets
// 256-byte aligned).  The arrival counters (one per sequence and group of heads_per_wg KV heads)
// come first and are sized for kMaxStepBatch sequences, so their place does not move with the
// batch: a workspace whose counters are zero stays valid for any batch with the same head
// layout.  Piece outputs and piece log-sum-exps follow.
struct StepWorkspace {
  uint64_t count_off, out_off, lse_off, bytes;
};
StepWorkspace step_workspace(const pkv_shape& s, int64_t groups, int heads_per_wg);

int check_step(const void* q, const void* k_new, const void* v_new, const void* k_pool,
               const void* v_pool, const int32_t* page_table, const int32_t* context_lens,
               float scale, const void* workspace, size_t workspace_bytes, uint64_t needed,
               const void* out, const float* lse_out, const pkv_shape* s, std::string& msg,
               int max_group = 16);

// The multi-query step: `s` is the caller's shape; the step runs over vs (num_q_heads = T x Hq),
// whose workspace needs `needed` bytes.
int check_multi_query_step(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* context_lens,
                           int32_t q_tokens, float scale, const void* workspace,
                           size_t workspace_bytes, uint64_t needed, const void* out,
                           const float* lse_out, const pkv_shape* s, const pkv_shape* vs,
                           std::string& msg);

// Most query tokens x GQA group of the multi-query step (eight waves of 16 head columns).
constexpr int kMaxMultiQueryColumns = 128;

int check_copy_pages(const void* k_pool, const void* v_pool, const int32_t* pairs,
                     int32_t n_pairs, const pkv_shape* s, std::string& msg);

int check_validate(const int32_t* page_table, const int32_t* context_lens, int32_t extra_tokens,
                   const int32_t* device_status, const pkv_shape* s, std::string& msg);

}  // namespace pkv
