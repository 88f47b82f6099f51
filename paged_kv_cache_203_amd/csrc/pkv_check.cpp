// Host-side argument checks (see pkv_check.h).  Every check runs before anything is enqueued:
// unsupported layouts, misaligned or aliased buffers and undersized workspaces are rejected up
// front rather than silently handled another way.
#include "pkv_check.h"

#include <cmath>
#include <cstdio>

namespace pkv {

namespace {

int fail(std::string& msg, int code, const char* text) {
  msg = text;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_F16: return 2;
    default: return 0;
  }
}

int check_shape(const pkv_shape* s, std::string& msg, int max_group) {
  if (!s) return fail(msg, PKV_EINVAL, "shape is NULL");
  if (s->batch < 0) return fail(msg, PKV_EINVAL, "batch must be >= 0");
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0)
    return fail(msg, PKV_EINVAL, "num_q_heads and num_kv_heads must be > 0");
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(msg, PKV_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (s->head_dim <= 0) return fail(msg, PKV_EINVAL, "head_dim must be > 0");
  if (s->page_size <= 0) return fail(msg, PKV_EINVAL, "page_size must be > 0");
  if (s->num_pages <= 0) return fail(msg, PKV_EINVAL, "num_pages must be > 0");
  if (s->max_pages_per_seq <= 0) return fail(msg, PKV_EINVAL, "max_pages_per_seq must be > 0");
  if (elem_bytes(s->dtype) == 0) return fail(msg, PKV_EUNSUPPORTED, "dtype must be f32, bf16 or f16");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(msg, PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (!is_pow2(s->page_size) || s->page_size < 16 || s->page_size > 256)
    return fail(msg, PKV_EUNSUPPORTED, "page_size must be a power of two in [16, 256]");
  if (s->num_q_heads / s->num_kv_heads > max_group)
    return fail(msg, PKV_EUNSUPPORTED,
                max_group == 16 ? "group size num_q_heads / num_kv_heads must be <= 16"
                                : "query columns per KV head (num_query_tokens x group) must be <= 128");
  // Tokens addressable by one row, and the largest in-page byte offset, must fit in int32.
  const int64_t row_tokens = int64_t(s->max_pages_per_seq) * s->page_size;
  if (row_tokens > INT32_MAX) return fail(msg, PKV_EINVAL, "max_pages_per_seq * page_size overflows int32");
  const int64_t page_bytes =
      int64_t(s->page_size) * s->num_kv_heads * s->head_dim * elem_bytes(s->dtype);
  if (page_bytes > INT32_MAX) return fail(msg, PKV_EUNSUPPORTED, "one page exceeds 2 GiB");
  if (int64_t(s->batch) * s->num_q_heads > INT32_MAX / 2)
    return fail(msg, PKV_EINVAL, "batch * num_q_heads too large");
  return PKV_OK;
}

Extents extents(const pkv_shape& s) {
  const uint64_t e = uint64_t(elem_bytes(s.dtype));
  Extents x;
  x.q = uint64_t(s.batch) * s.num_q_heads * s.head_dim * e;
  x.out = x.q;
  x.pool = uint64_t(s.num_pages) * s.page_size * s.num_kv_heads * s.head_dim * e;
  x.new_rows = uint64_t(s.batch) * s.num_kv_heads * s.head_dim * e;
  x.table = uint64_t(s.batch) * s.max_pages_per_seq * 4;
  x.lens = uint64_t(s.batch) * 4;
  return x;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

static int check_attention_inputs(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, const int32_t* context_lens,
                                  float scale, std::string& msg) {
  if (!q || !k_pool || !v_pool || !page_table || !context_lens)
    return fail(msg, PKV_EINVAL, "q, k_pool, v_pool, page_table and context_lens must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(msg, PKV_EUNSUPPORTED, "q, k_pool and v_pool must be 16-byte aligned");
  if (!aligned(page_table, 4) || !aligned(context_lens, 4))
    return fail(msg, PKV_EINVAL, "page_table and context_lens must be 4-byte aligned");
  if (!std::isfinite(scale)) return fail(msg, PKV_EINVAL, "scale must be finite");
  return PKV_OK;
}

int check_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                 const int32_t* context_lens, float scale, const void* out, const pkv_shape* s,
                 std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (s->batch == 0) return PKV_OK;
  rc = check_attention_inputs(q, k_pool, v_pool, page_table, context_lens, scale, msg);
  if (rc) return rc;
  if (!out) return fail(msg, PKV_EINVAL, "out must be non-NULL");
  if (!aligned(out, 16)) return fail(msg, PKV_EUNSUPPORTED, "out must be 16-byte aligned");
  const Extents x = extents(*s);
  if (overlaps(out, x.out, q, x.q) || overlaps(out, x.out, k_pool, x.pool) ||
      overlaps(out, x.out, v_pool, x.pool) || overlaps(out, x.out, page_table, x.table) ||
      overlaps(out, x.out, context_lens, x.lens))
    return fail(msg, PKV_EINVAL, "out overlaps an input");
  return PKV_OK;
}

int32_t partitions_needed(const pkv_shape& s, int32_t partition_tokens) {
  const int64_t row_tokens = int64_t(s.max_pages_per_seq) * s.page_size;
  return int32_t((row_tokens + partition_tokens - 1) / partition_tokens);
}

int check_partial(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                  const int32_t* context_lens, float scale, int32_t partition_tokens,
                  const float* partial_out, const float* partial_lse, int32_t max_partitions,
                  const pkv_shape* s, std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (partition_tokens <= 0 || partition_tokens % s->page_size != 0)
    return fail(msg, PKV_EINVAL, "partition_tokens must be a positive multiple of page_size");
  if (max_partitions <= 0) return fail(msg, PKV_EINVAL, "max_partitions must be > 0");
  if (max_partitions < partitions_needed(*s, partition_tokens))
    return fail(msg, PKV_EWORKSPACE,
                "max_partitions < ceil(max_pages_per_seq * page_size / partition_tokens)");
  if (s->batch == 0) return PKV_OK;
  rc = check_attention_inputs(q, k_pool, v_pool, page_table, context_lens, scale, msg);
  if (rc) return rc;
  if (!partial_out || !partial_lse)
    return fail(msg, PKV_EINVAL, "partial_out and partial_lse must be non-NULL");
  if (!aligned(partial_out, 16) || !aligned(partial_lse, 4))
    return fail(msg, PKV_EUNSUPPORTED, "partial_out must be 16-byte and partial_lse 4-byte aligned");
  const Extents x = extents(*s);
  const uint64_t rows = uint64_t(s->batch) * s->num_q_heads * uint64_t(max_partitions);
  const uint64_t po = rows * s->head_dim * 4, pl = rows * 4;
  const void* ins[5] = {q, k_pool, v_pool, page_table, context_lens};
  const uint64_t ins_n[5] = {x.q, x.pool, x.pool, x.table, x.lens};
  for (int i = 0; i < 5; ++i)
    if (overlaps(partial_out, po, ins[i], ins_n[i]) || overlaps(partial_lse, pl, ins[i], ins_n[i]))
      return fail(msg, PKV_EINVAL, "partial buffers overlap an input");
  if (overlaps(partial_out, po, partial_lse, pl))
    return fail(msg, PKV_EINVAL, "partial_out overlaps partial_lse");
  return PKV_OK;
}

int check_merge(const float* partial_out, const float* partial_lse, const int32_t* context_lens,
                int32_t partition_tokens, int32_t max_partitions, const void* out,
                const float* lse_out, const pkv_shape* s, std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (partition_tokens <= 0 || partition_tokens % s->page_size != 0)
    return fail(msg, PKV_EINVAL, "partition_tokens must be a positive multiple of page_size");
  if (max_partitions <= 0) return fail(msg, PKV_EINVAL, "max_partitions must be > 0");
  if (max_partitions < partitions_needed(*s, partition_tokens))
    return fail(msg, PKV_EWORKSPACE,
                "max_partitions < ceil(max_pages_per_seq * page_size / partition_tokens)");
  if (s->batch == 0) return PKV_OK;
  if (!partial_out || !partial_lse || !context_lens || !out)
    return fail(msg, PKV_EINVAL, "partial_out, partial_lse, context_lens and out must be non-NULL");
  if (!aligned(partial_out, 16) || !aligned(out, 16))
    return fail(msg, PKV_EUNSUPPORTED, "partial_out and out must be 16-byte aligned");
  if (!aligned(partial_lse, 4) || !aligned(context_lens, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(msg, PKV_EINVAL, "partial_lse, context_lens and lse_out must be 4-byte aligned");
  const Extents x = extents(*s);
  const uint64_t rows = uint64_t(s->batch) * s->num_q_heads * uint64_t(max_partitions);
  const uint64_t po = rows * s->head_dim * 4, pl = rows * 4;
  const uint64_t lo = uint64_t(s->batch) * s->num_q_heads * 4;
  if (overlaps(out, x.out, partial_out, po) || overlaps(out, x.out, partial_lse, pl) ||
      overlaps(out, x.out, context_lens, x.lens))
    return fail(msg, PKV_EINVAL, "out overlaps an input");
  if (lse_out && (overlaps(lse_out, lo, partial_out, po) || overlaps(lse_out, lo, partial_lse, pl) ||
                  overlaps(lse_out, lo, out, x.out) || overlaps(lse_out, lo, context_lens, x.lens)))
    return fail(msg, PKV_EINVAL, "lse_out overlaps another buffer");
  return PKV_OK;
}

int check_cascade(const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* prefix_pages, int32_t prefix_tokens, const int32_t* page_table,
                  const int32_t* context_lens, float scale, int32_t partition_tokens,
                  const float* partial_out, const float* partial_lse, int32_t max_partitions,
                  const void* out, const float* lse_out, const pkv_shape* s, std::string& msg) {
  int rc = check_partial(q, k_pool, v_pool, page_table, context_lens, scale, partition_tokens,
                         partial_out, partial_lse, max_partitions, s, msg);
  if (rc) return rc;
  if (s->dtype != PKV_BF16 && s->dtype != PKV_F16)
    return fail(msg, PKV_EUNSUPPORTED, "the shared-prefix path supports bf16 and f16 only");
  if (partition_tokens % kPrefixBlock != 0)
    return fail(msg, PKV_EUNSUPPORTED, "partition_tokens must be a multiple of 64");
  if (partition_tokens / s->page_size > kMaxPrefixPageIds)
    return fail(msg, PKV_EUNSUPPORTED, "partition_tokens / page_size must be <= 512");
  const int64_t capacity = int64_t(s->max_pages_per_seq) * s->page_size;
  if (prefix_tokens < 0 || prefix_tokens % partition_tokens != 0 || prefix_tokens > capacity)
    return fail(msg, PKV_EINVAL,
                "prefix_tokens must be a multiple of partition_tokens in [0, max_pages_per_seq * page_size]");
  if (s->batch == 0) return PKV_OK;
  if (prefix_tokens > 0 && (!prefix_pages || !aligned(prefix_pages, 4)))
    return fail(msg, PKV_EINVAL, "prefix_pages must be non-NULL and 4-byte aligned");
  if (!out) return fail(msg, PKV_EINVAL, "out must be non-NULL");
  if (!aligned(out, 16)) return fail(msg, PKV_EUNSUPPORTED, "out must be 16-byte aligned");
  if (lse_out && !aligned(lse_out, 4)) return fail(msg, PKV_EINVAL, "lse_out must be 4-byte aligned");
  const Extents x = extents(*s);
  const uint64_t rows = uint64_t(s->batch) * s->num_q_heads * uint64_t(max_partitions);
  const uint64_t po = rows * s->head_dim * 4, pl = rows * 4;
  const uint64_t lo = uint64_t(s->batch) * s->num_q_heads * 4;
  const uint64_t pp = uint64_t(prefix_tokens / s->page_size) * 4;
  if (overlaps(partial_out, po, prefix_pages, pp) || overlaps(partial_lse, pl, prefix_pages, pp))
    return fail(msg, PKV_EINVAL, "partial buffers overlap prefix_pages");
  const void* ins[7] = {q, k_pool, v_pool, page_table, context_lens, partial_out, partial_lse};
  const uint64_t ins_n[7] = {x.q, x.pool, x.pool, x.table, x.lens, po, pl};
  for (int i = 0; i < 7; ++i) {
    if (overlaps(out, x.out, ins[i], ins_n[i])) return fail(msg, PKV_EINVAL, "out overlaps another buffer");
    if (lse_out && overlaps(lse_out, lo, ins[i], ins_n[i]))
      return fail(msg, PKV_EINVAL, "lse_out overlaps another buffer");
  }
  if (overlaps(out, x.out, prefix_pages, pp) || (lse_out && overlaps(lse_out, lo, prefix_pages, pp)))
    return fail(msg, PKV_EINVAL, "an output overlaps prefix_pages");
  if (lse_out && overlaps(lse_out, lo, out, x.out)) return fail(msg, PKV_EINVAL, "lse_out overlaps out");
  return PKV_OK;
}

int check_multi_query(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* page_table, const int32_t* context_lens, int32_t q_tokens,
                      float scale, int32_t partition_tokens, const float* partial_out,
                      const float* partial_lse, int32_t max_partitions, const void* out,
                      const float* lse_out, const pkv_shape* s, std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (q_tokens < 1) return fail(msg, PKV_EINVAL, "num_query_tokens must be >= 1");
  if (int64_t(s->batch) * q_tokens * s->num_q_heads > INT32_MAX / 2)
    return fail(msg, PKV_EINVAL, "batch * num_query_tokens * num_q_heads too large");
  if (s->dtype != PKV_BF16 && s->dtype != PKV_F16)
    return fail(msg, PKV_EUNSUPPORTED, "multi-query decode supports bf16 and f16 only");
  if (partition_tokens <= 0 || partition_tokens % s->page_size != 0 ||
      partition_tokens % kPrefixBlock != 0)
    return fail(msg, PKV_EUNSUPPORTED, "partition_tokens must be a positive multiple of 64 and of page_size");
  if (partition_tokens / s->page_size > kMaxPrefixPageIds)
    return fail(msg, PKV_EUNSUPPORTED, "partition_tokens / page_size must be <= 512");
  if (max_partitions <= 0) return fail(msg, PKV_EINVAL, "max_partitions must be > 0");
  if (max_partitions < partitions_needed(*s, partition_tokens))
    return fail(msg, PKV_EWORKSPACE,
                "max_partitions < ceil(max_pages_per_seq * page_size / partition_tokens)");
  if (s->batch == 0) return PKV_OK;
  rc = check_attention_inputs(q, k_pool, v_pool, page_table, context_lens, scale, msg);
  if (rc) return rc;
  if (!partial_out || !partial_lse || !out)
    return fail(msg, PKV_EINVAL, "partial_out, partial_lse and out must be non-NULL");
  if (!aligned(partial_out, 16) || !aligned(out, 16))
    return fail(msg, PKV_EUNSUPPORTED, "partial_out and out must be 16-byte aligned");
  if (!aligned(partial_lse, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(msg, PKV_EINVAL, "partial_lse and lse_out must be 4-byte aligned");
  const Extents x = extents(*s);
  const uint64_t rows = uint64_t(s->batch) * q_tokens * s->num_q_heads;
  const uint64_t qn = rows * s->head_dim * elem_bytes(s->dtype);
  const uint64_t po = rows * uint64_t(max_partitions) * s->head_dim * 4;
  const uint64_t pl = rows * uint64_t(max_partitions) * 4;
  const uint64_t lo = rows * 4;
  const void* ins[5] = {q, k_pool, v_pool, page_table, context_lens};
  const uint64_t ins_n[5] = {qn, x.pool, x.pool, x.table, x.lens};
  const void* outs[4] = {partial_out, partial_lse, out, lse_out};
  const uint64_t outs_n[4] = {po, pl, qn, lse_out ? lo : 0};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], outs_n[i], ins[j], ins_n[j]))
        return fail(msg, PKV_EINVAL, "an output or the partials overlap an input");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs_n[i], outs[j], outs_n[j]))
        return fail(msg, PKV_EINVAL, "partials, out and lse_out must not overlap");
  }
  return PKV_OK;
}

int check_append(const void* k_new, const void* v_new, const void* k_pool, const void* v_pool,
                 const int32_t* page_table, const int32_t* context_lens, const pkv_shape* s,
                 std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (s->batch == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !page_table || !context_lens)
    return fail(msg, PKV_EINVAL, "every pointer must be non-NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(msg, PKV_EUNSUPPORTED, "k_new, v_new and the pools must be 16-byte aligned");
  if (!aligned(page_table, 4) || !aligned(context_lens, 4))
    return fail(msg, PKV_EINVAL, "page_table and context_lens must be 4-byte aligned");
  const Extents x = extents(*s);
  if (overlaps(k_pool, x.pool, v_pool, x.pool)) return fail(msg, PKV_EINVAL, "k_pool overlaps v_pool");
  const void* ins[4] = {k_new, v_new, page_table, context_lens};
  const uint64_t ins_n[4] = {x.new_rows, x.new_rows, x.table, x.lens};
  for (int i = 0; i < 4; ++i)
    if (overlaps(k_pool, x.pool, ins[i], ins_n[i]) || overlaps(v_pool, x.pool, ins[i], ins_n[i]))
      return fail(msg, PKV_EINVAL, "a pool overlaps an input of the append");
  return PKV_OK;
}

StepWorkspace step_workspace(const pkv_shape& s, int64_t groups, int heads_per_wg) {
  auto up = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
  const uint64_t pieces = uint64_t(groups) + uint64_t(s.batch);
  const uint64_t head_groups = uint64_t(s.num_kv_heads / heads_per_wg);
  StepWorkspace w;
  w.count_off = 0;
  w.out_off = up(uint64_t(kMaxStepBatch) * head_groups * 8);
  w.lse_off = w.out_off + up(pieces * s.num_q_heads * s.head_dim * 4);
  w.bytes = w.lse_off + up(pieces * s.num_q_heads * 4);
  return w;
}

int check_step(const void* q, const void* k_new, const void* v_new, const void* k_pool,
               const void* v_pool, const int32_t* page_table, const int32_t* context_lens,
               float scale, const void* workspace, size_t workspace_bytes, uint64_t needed,
               const void* out, const float* lse_out, const pkv_shape* s, std::string& msg,
               int max_group) {
  int rc = check_shape(s, msg, max_group);
  if (rc) return rc;
  if (s->batch > kMaxStepBatch)
    return fail(msg, PKV_EUNSUPPORTED, "batch must be <= 4096 for the decode step");
  if (s->num_q_heads > kMaxStepHeads)
    return fail(msg, PKV_EUNSUPPORTED, "num_q_heads must be <= 1024 for the decode step");
  {
    // The step's work split counts 4 units per 16-token tile plus up to 24 per sequence in int32.
    const int64_t tiles = (int64_t(s->max_pages_per_seq) * s->page_size + 1 + 15) / 16;
    if (int64_t(s->batch) * (4 * tiles + 24) >= (int64_t(1) << 31))
      return fail(msg, PKV_EUNSUPPORTED, "batch * page-table capacity too large for the decode step");
  }
  if (s->batch == 0) return PKV_OK;
  rc = check_attention_inputs(q, k_pool, v_pool, page_table, context_lens, scale, msg);
  if (rc) return rc;
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(msg, PKV_EINVAL, "k_new and v_new must both be given or both be NULL");
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16)))
    return fail(msg, PKV_EUNSUPPORTED, "k_new and v_new must be 16-byte aligned");
  if (!out) return fail(msg, PKV_EINVAL, "out must be non-NULL");
  if (!aligned(out, 16)) return fail(msg, PKV_EUNSUPPORTED, "out must be 16-byte aligned");
  if (lse_out && !aligned(lse_out, 4)) return fail(msg, PKV_EINVAL, "lse_out must be 4-byte aligned");
  if (!workspace) return fail(msg, PKV_EINVAL, "workspace must be non-NULL");
  if (!aligned(workspace, 16)) return fail(msg, PKV_EINVAL, "workspace must be 16-byte aligned");
  const Extents x = extents(*s);
  const uint64_t lo = uint64_t(s->batch) * s->num_q_heads * 4;
  const void* ins[7] = {q, k_pool, v_pool, page_table, context_lens, k_new, v_new};
  const uint64_t ins_n[7] = {x.q, x.pool, x.pool, x.table, x.lens, x.new_rows, x.new_rows};
  for (int i = 0; i < 7; ++i) {
    if (overlaps(out, x.out, ins[i], ins_n[i])) return fail(msg, PKV_EINVAL, "out overlaps an input");
    if (overlaps(workspace, workspace_bytes, ins[i], ins_n[i]))
      return fail(msg, PKV_EINVAL, "workspace overlaps an input");
    if (lse_out && overlaps(lse_out, lo, ins[i], ins_n[i]))
      return fail(msg, PKV_EINVAL, "lse_out overlaps an input");
  }
  if (overlaps(out, x.out, workspace, workspace_bytes) || (lse_out && overlaps(lse_out, lo, workspace, workspace_bytes)) ||
      (lse_out && overlaps(lse_out, lo, out, x.out)))
    return fail(msg, PKV_EINVAL, "out, lse_out and workspace must not overlap");
  if (k_new) {
    if (overlaps(k_pool, x.pool, v_pool, x.pool)) return fail(msg, PKV_EINVAL, "k_pool overlaps v_pool");
    const void* rd[4] = {k_new, v_new, page_table, context_lens};
    const uint64_t rd_n[4] = {x.new_rows, x.new_rows, x.table, x.lens};
    for (int i = 0; i < 4; ++i)
      if (overlaps(k_pool, x.pool, rd[i], rd_n[i]) || overlaps(v_pool, x.pool, rd[i], rd_n[i]))
        return fail(msg, PKV_EINVAL, "a pool overlaps an input of the append");
  }
  if (needed == 0) return fail(msg, PKV_ELAUNCH, "no device available to size the workspace");
  if (workspace_bytes < needed)
    return fail(msg, PKV_EWORKSPACE, "workspace smaller than pkv_decode_step_workspace_bytes() "
                                      "(pkv_multi_query_step_workspace_bytes() for the multi-query step)");
  return PKV_OK;
}

int check_rope_tables(const void* k_new, const float* rope_cos, const float* rope_sin,
                      int32_t rope_positions, const void* out, const float* lse_out,
                      const void* workspace, size_t workspace_bytes, const pkv_shape* s,
                      std::string& msg) {
  if (!k_new) return fail(msg, PKV_EINVAL, "the rotary embedding needs the appended rows");
  if (rope_positions <= 0) return fail(msg, PKV_EINVAL, "rope_positions must be > 0");
  if (!rope_cos || !rope_sin) return fail(msg, PKV_EINVAL, "rope_cos and rope_sin must be non-NULL");
  if (!aligned(rope_cos, 16) || !aligned(rope_sin, 16))
    return fail(msg, PKV_EUNSUPPORTED, "rope_cos and rope_sin must be 16-byte aligned");
  const Extents x = extents(*s);
  const uint64_t tab = uint64_t(rope_positions) * (s->head_dim / 2) * 4;
  const uint64_t lo = uint64_t(s->batch) * s->num_q_heads * 4;
  for (const void* t : {static_cast<const void*>(rope_cos), static_cast<const void*>(rope_sin)})
    if (overlaps(t, tab, out, x.out) || (lse_out && overlaps(t, tab, lse_out, lo)) ||
        overlaps(t, tab, workspace, workspace_bytes))
      return fail(msg, PKV_EINVAL, "the rotary cache overlaps an output or the workspace");
  return PKV_OK;
}

int check_rope_append(const void* q, const void* k_new, const void* v_new, const void* k_pool,
                      const void* v_pool, const int32_t* page_table, const int32_t* context_lens,
                      const float* rope_cos, const float* rope_sin, int32_t rope_positions,
                      const void* q_out, const pkv_shape* s, std::string& msg) {
  int rc = check_append(k_new, v_new, k_pool, v_pool, page_table, context_lens, s, msg);
  if (rc) return rc;
  if (rope_positions <= 0) return fail(msg, PKV_EINVAL, "rope_positions must be > 0");
  if (s->batch == 0) return PKV_OK;
  if (!q || !q_out || !rope_cos || !rope_sin)
    return fail(msg, PKV_EINVAL, "q, q_out, rope_cos and rope_sin must be non-NULL");
  if (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16))
    return fail(msg, PKV_EUNSUPPORTED, "q, q_out, rope_cos and rope_sin must be 16-byte aligned");
  const Extents x = extents(*s);
  const uint64_t tab = uint64_t(rope_positions) * (s->head_dim / 2) * 4;
  const void* ins[9] = {q, k_new, v_new, k_pool, v_pool, page_table, context_lens, rope_cos, rope_sin};
  const uint64_t ins_n[9] = {x.q, x.new_rows, x.new_rows, x.pool, x.pool, x.table, x.lens, tab, tab};
  for (int i = 0; i < 9; ++i)
    if (overlaps(q_out, x.q, ins[i], ins_n[i])) return fail(msg, PKV_EINVAL, "q_out overlaps another buffer");
  for (int i = 3; i < 5; ++i)
    for (int j : {0, 7, 8})
      if (overlaps(ins[i], ins_n[i], ins[j], ins_n[j]))
        return fail(msg, PKV_EINVAL, "a pool overlaps q or the rotary cache");
  return PKV_OK;
}

int check_multi_query_step(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* context_lens,
                           int32_t q_tokens, float scale, const void* workspace,
                           size_t workspace_bytes, uint64_t needed, const void* out,
                           const float* lse_out, const pkv_shape* s, const pkv_shape* vs,
                           std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (q_tokens < 1) return fail(msg, PKV_EINVAL, "num_query_tokens must be >= 1");
  if (s->dtype != PKV_BF16 && s->dtype != PKV_F16)
    return fail(msg, PKV_EUNSUPPORTED, "the multi-query step supports bf16 and f16 only");
  if (int64_t(q_tokens) * (s->num_q_heads / s->num_kv_heads) > kMaxMultiQueryColumns)
    return fail(msg, PKV_EUNSUPPORTED,
                "num_query_tokens * (num_q_heads / num_kv_heads) must be <= 128 for the multi-query step");
  return check_step(q, nullptr, nullptr, k_pool, v_pool, page_table, context_lens, scale, workspace,
                    workspace_bytes, needed, out, lse_out, vs, msg, kMaxMultiQueryColumns);
}

int check_copy_pages(const void* k_pool, const void* v_pool, const int32_t* pairs,
                     int32_t n_pairs, const pkv_shape* s, std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (n_pairs < 0) return fail(msg, PKV_EINVAL, "n_pairs must be >= 0");
  if (n_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !pairs)
    return fail(msg, PKV_EINVAL, "k_pool, v_pool and pairs must be non-NULL");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(msg, PKV_EUNSUPPORTED, "the pools must be 16-byte aligned");
  if (!aligned(pairs, 4)) return fail(msg, PKV_EINVAL, "pairs must be 4-byte aligned");
  const Extents x = extents(*s);
  if (overlaps(k_pool, x.pool, v_pool, x.pool)) return fail(msg, PKV_EINVAL, "k_pool overlaps v_pool");
  const uint64_t pn = uint64_t(n_pairs) * 8;
  if (overlaps(pairs, pn, k_pool, x.pool) || overlaps(pairs, pn, v_pool, x.pool))
    return fail(msg, PKV_EINVAL, "pairs overlap a pool");
  return PKV_OK;
}

int check_validate(const int32_t* page_table, const int32_t* context_lens, int32_t extra_tokens,
                   const int32_t* device_status, const pkv_shape* s, std::string& msg) {
  int rc = check_shape(s, msg);
  if (rc) return rc;
  if (extra_tokens < 0) return fail(msg, PKV_EINVAL, "extra_tokens must be >= 0");
  if (!device_status) return fail(msg, PKV_EINVAL, "device_status must be non-NULL");
  if (!aligned(device_status, 4)) return fail(msg, PKV_EINVAL, "device_status must be 4-byte aligned");
  if (s->batch == 0) return PKV_OK;
  if (!page_table || !context_lens)
    return fail(msg, PKV_EINVAL, "page_table and context_lens must be non-NULL");
  if (!aligned(page_table, 4) || !aligned(context_lens, 4))
    return fail(msg, PKV_EINVAL, "page_table and context_lens must be 4-byte aligned");
  return PKV_OK;
}

}  // namespace pkv
