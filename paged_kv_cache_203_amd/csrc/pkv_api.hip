// C-ABI entry points of libpkv (declared in include/pkv.h): host-side checks, then one launch on
// the caller's stream.  No allocation and no synchronisation; the only state kept between calls
// is the decode step's call generation (one counter per process).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <string>

#include "../../include/pkv.h"
#include "pkv_arrival.h"
#include "pkv_check.h"
#include "pkv_launch.h"

namespace {

thread_local std::string g_last_error;

// Generation of the decode step's calls in this process (pkv_arrival.h): every call takes the
// next one, so a counter that an earlier call left behind counts from zero again.
std::atomic<uint32_t> g_step_generation{0};

uint32_t take_generation() {
  uint32_t g = g_step_generation.load(std::memory_order_relaxed), n;
  do {
    n = pkv::next_generation(g);
  } while (!g_step_generation.compare_exchange_weak(g, n, std::memory_order_relaxed));
  return n;
}

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int log2_exact(int32_t x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

int group_pad(int g) { return g <= 4 ? 4 : (g <= 8 ? 8 : 16); }

// Largest divisor of hkv that also divides the decode workgroup's wave count.
int heads_per_workgroup(int hkv) {
  const int waves = pkv::decode_waves();
  int best = 1;
  for (int h = 1; h <= waves; ++h)
    if (hkv % h == 0 && waves % h == 0) best = h;
  return best;
}

// KV heads per workgroup of the balanced decode step: as many as divide both hkv and the wave
// count, then halved while some wave would hold more than `per_wave` query heads; with fewer
// heads per workgroup, the waves that share a KV head split its query heads.  With PV on the
// matrix cores (16-bit K/V, head_dim 128) a wave's output tile has 16 query-head columns
// whatever the group, so up to 16 heads per wave cost no more registers or matrix-core work
// than 4; with PV on the VALU, 8- and 16-column accumulators do not fit the register budget
// without spills, so the limit there is 4.
int step_heads_per_workgroup(int hkv, int group, int per_wave) {
  const int waves = pkv::decode_waves();
  int h = heads_per_workgroup(hkv);
  while (h > 1) {
    const int wph = waves / h;
    const int gw = (group + wph - 1) / wph;
    const bool split = wph > 1 && (wph - 1) * gw < group;
    if ((split ? gw : group) <= per_wave) break;
    h /= 2;
  }
  return h;
}
int step_heads_per_workgroup(const pkv_shape& s) {
  const int per_wave = s.dtype != PKV_F32 && s.head_dim == 128 ? 16 : 4;
  return step_heads_per_workgroup(s.num_kv_heads, s.num_q_heads / s.num_kv_heads, per_wave);
}

// Workgroup ranges of the balanced decode step on the current device: one 8-wave workgroup per
// compute unit, shared among the KV-head groups.  0 when no device is available.
int64_t step_groups(const pkv_shape& s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int nhg = s.num_kv_heads / step_heads_per_workgroup(s);
  return cus / nhg > 0 ? cus / nhg : 1;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return set_error(PKV_ELAUNCH, std::string(what) + ": " + hipGetErrorString(e));
}

pkv::DecodeParams decode_params(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* page_table, const int32_t* context_lens,
                                float scale, const pkv_shape& s) {
  pkv::DecodeParams p{};
  const int e = pkv::elem_bytes(s.dtype);
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.page_table = page_table;
  p.context_lens = context_lens;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  p.batch = s.batch;
  p.hq = s.num_q_heads;
  p.hkv = s.num_kv_heads;
  p.group = s.num_q_heads / s.num_kv_heads;
  p.num_pages = s.num_pages;
  p.max_pages = s.max_pages_per_seq;
  p.page_shift = log2_exact(s.page_size);
  p.capacity = s.max_pages_per_seq * s.page_size;
  p.tok_stride = s.num_kv_heads * s.head_dim * e;
  p.page_stride = int64_t(s.page_size) * p.tok_stride;
  return p;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

size_t pkv_partial_workspace_bytes(const pkv_shape* shape, int32_t max_partitions) {
  std::string msg;
  if (pkv::check_shape(shape, msg) != PKV_OK || max_partitions <= 0) return 0;
  const uint64_t rows = uint64_t(shape->batch) * shape->num_q_heads * uint64_t(max_partitions);
  return size_t(rows * shape->head_dim * 4 + rows * 4);
}

int pkv_paged_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* page_table, const int32_t* context_lens,
                               float scale, void* out, const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_decode(q, k_pool, v_pool, page_table, context_lens, scale, out, shape, msg);
  if (rc) return set_error(rc, "pkv_paged_decode_attention: " + msg);
  if (shape->batch == 0) return PKV_OK;
  pkv::DecodeParams p = decode_params(q, k_pool, v_pool, page_table, context_lens, scale, *shape);
  p.out = out;
  p.partition_tokens = p.capacity;
  p.max_partitions = 1;
  p.heads_per_wg = 1;   // one KV head per workgroup: its waves share the whole sequence
  (void)hipGetLastError();
  return launch_status(pkv::launch_decode(p, shape->dtype, shape->head_dim, group_pad(p.group),
                                          false, static_cast<hipStream_t>(stream)),
                       "pkv_paged_decode_attention");
}

int pkv_paged_decode_attention_partial(const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* page_table, const int32_t* context_lens,
                                       float scale, int32_t partition_tokens,
                                       float* partial_out, float* partial_lse,
                                       int32_t max_partitions, const pkv_shape* shape,
                                       void* stream) {
  std::string msg;
  const int rc = pkv::check_partial(q, k_pool, v_pool, page_table, context_lens, scale,
                                    partition_tokens, partial_out, partial_lse, max_partitions,
                                    shape, msg);
  if (rc) return set_error(rc, "pkv_paged_decode_attention_partial: " + msg);
  if (shape->batch == 0) return PKV_OK;
  pkv::DecodeParams p = decode_params(q, k_pool, v_pool, page_table, context_lens, scale, *shape);
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.partition_tokens = partition_tokens;
  p.max_partitions = max_partitions;
  p.heads_per_wg = heads_per_workgroup(p.hkv);   // whole pages per workgroup
  (void)hipGetLastError();
  return launch_status(pkv::launch_decode(p, shape->dtype, shape->head_dim, group_pad(p.group),
                                          true, static_cast<hipStream_t>(stream)),
                       "pkv_paged_decode_attention_partial");
}

int pkv_paged_decode_cascade(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* prefix_pages, int32_t prefix_tokens,
                             const int32_t* page_table, const int32_t* context_lens, float scale,
                             int32_t partition_tokens, float* partial_out, float* partial_lse,
                             int32_t max_partitions, void* out, float* lse_out,
                             const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_cascade(q, k_pool, v_pool, prefix_pages, prefix_tokens, page_table,
                                    context_lens, scale, partition_tokens, partial_out,
                                    partial_lse, max_partitions, out, lse_out, shape, msg);
  if (rc) return set_error(rc, "pkv_paged_decode_cascade: " + msg);
  if (shape->batch == 0) return PKV_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  pkv::DecodeParams d = decode_params(q, k_pool, v_pool, page_table, context_lens, scale, *shape);
  (void)hipGetLastError();

  pkv::PrefixParams pp{};
  pp.q = q;
  pp.k_pool = k_pool;
  pp.v_pool = v_pool;
  pp.prefix_pages = prefix_pages;
  pp.context_lens = context_lens;
  pp.partial_out = partial_out;
  pp.partial_lse = partial_lse;
  pp.scale_log2 = d.scale_log2;
  pp.batch = d.batch;
  pp.hq = d.hq;
  pp.hkv = d.hkv;
  pp.group = d.group;
  pp.num_pages = d.num_pages;
  pp.page_shift = d.page_shift;
  pp.capacity = d.capacity;
  pp.prefix_tokens = prefix_tokens;
  pp.partition_tokens = partition_tokens;
  pp.max_partitions = max_partitions;
  pp.tok_stride = d.tok_stride;
  pp.page_stride = d.page_stride;
  // The suffix partitions (from partition prefix_tokens / P on) and the prefix partitions in one
  // grid, then the merge.
  d.partial_out = partial_out;
  d.partial_lse = partial_lse;
  d.partition_tokens = partition_tokens;
  d.max_partitions = max_partitions;
  d.part_begin = prefix_tokens / partition_tokens;
  d.heads_per_wg = heads_per_workgroup(d.hkv);
  const int r = launch_status(pkv::launch_cascade(d, pp, shape->dtype, shape->head_dim,
                                                  group_pad(d.group), st),
                              "pkv_paged_decode_cascade (partitions)");
  if (r) return r;

  pkv::MergeParams m{};
  m.partial_out = partial_out;
  m.partial_lse = partial_lse;
  m.context_lens = context_lens;
  m.out = out;
  m.lse_out = lse_out;
  m.batch = shape->batch;
  m.hq = shape->num_q_heads;
  m.partition_tokens = partition_tokens;
  m.max_partitions = max_partitions;
  m.capacity = d.capacity;
  return launch_status(pkv::launch_merge(m, shape->dtype, shape->head_dim, st),
                       "pkv_paged_decode_cascade (merge)");
}

int pkv_paged_decode_multi_query(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* page_table, const int32_t* context_lens,
                                 int32_t num_query_tokens, float scale, int32_t partition_tokens,
                                 float* partial_out, float* partial_lse, int32_t max_partitions,
                                 void* out, float* lse_out, const pkv_shape* shape,
                                 void* stream) {
  std::string msg;
  const int rc = pkv::check_multi_query(q, k_pool, v_pool, page_table, context_lens,
                                        num_query_tokens, scale, partition_tokens, partial_out,
                                        partial_lse, max_partitions, out, lse_out, shape, msg);
  if (rc) return set_error(rc, "pkv_paged_decode_multi_query: " + msg);
  if (shape->batch == 0) return PKV_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const pkv::DecodeParams d = decode_params(q, k_pool, v_pool, page_table, context_lens, scale, *shape);
  (void)hipGetLastError();
  // 1. Every (sequence, KV head, partition): its G x T query rows against the partition's
  //    tokens on the matrix cores, query j masked past its own position.
  pkv::PrefixParams pp{};
  pp.q = q;
  pp.k_pool = k_pool;
  pp.v_pool = v_pool;
  pp.context_lens = context_lens;
  pp.partial_out = partial_out;
  pp.partial_lse = partial_lse;
  pp.scale_log2 = d.scale_log2;
  pp.batch = d.batch;
  pp.hq = d.hq;
  pp.hkv = d.hkv;
  pp.group = d.group;
  pp.num_pages = d.num_pages;
  pp.page_shift = d.page_shift;
  pp.capacity = d.capacity;
  pp.partition_tokens = partition_tokens;
  pp.max_partitions = max_partitions;
  pp.tok_stride = d.tok_stride;
  pp.page_stride = d.page_stride;
  pp.page_table = page_table;
  pp.max_pages = d.max_pages;
  pp.q_tokens = num_query_tokens;
  int r = launch_status(pkv::launch_prefix(pp, shape->dtype, shape->head_dim, st),
                        "pkv_paged_decode_multi_query (partitions)");
  if (r) return r;
  // 2. The merge of each (sequence, query token)'s partitions.
  pkv::MergeParams m{};
  m.partial_out = partial_out;
  m.partial_lse = partial_lse;
  m.context_lens = context_lens;
  m.out = out;
  m.lse_out = lse_out;
  m.batch = shape->batch;
  m.hq = shape->num_q_heads;
  m.partition_tokens = partition_tokens;
  m.max_partitions = max_partitions;
  m.capacity = d.capacity;
  m.q_tokens = num_query_tokens;
  return launch_status(pkv::launch_merge(m, shape->dtype, shape->head_dim, st),
                       "pkv_paged_decode_multi_query (merge)");
}

size_t pkv_decode_step_workspace_bytes(const pkv_shape* shape) {
  std::string msg;
  if (pkv::check_shape(shape, msg) != PKV_OK) return 0;
  const int64_t groups = step_groups(*shape);
  if (groups == 0) return 0;
  return size_t(pkv::step_workspace(*shape, groups, step_heads_per_workgroup(*shape)).bytes);
}

namespace {
// The shape the step runs over: the caller's, or for the multi-query step (q_tokens = T > 1) the
// same with T x num_q_heads heads (query token j of query head h is head (h / G) x T G + j G + h % G).
pkv_shape step_shape(const pkv_shape& s, int32_t q_tokens) {
  pkv_shape v = s;
  if (q_tokens > 1) v.num_q_heads = s.num_q_heads * q_tokens;
  return v;
}

int decode_step(const char* name, const void* q, const void* k_new, const void* v_new,
                void* k_pool, void* v_pool, const int32_t* page_table,
                const int32_t* context_lens, const float* rope_cos, const float* rope_sin,
                int32_t rope_positions, float scale, void* workspace, size_t workspace_bytes,
                void* out, float* lse_out, const pkv_shape* user_shape, void* stream,
                int32_t q_tokens = 1) {
  std::string msg;
  int rc = pkv::check_shape(user_shape, msg);
  if (rc) return set_error(rc, std::string(name) + ": " + msg);
  const pkv_shape vshape = step_shape(*user_shape, q_tokens);
  const pkv_shape* shape = &vshape;
  const int64_t groups = shape->batch ? step_groups(*shape) : 1;
  const pkv::StepWorkspace ws =
      pkv::step_workspace(*shape, groups ? groups : 1, step_heads_per_workgroup(*shape));
  if (q_tokens > 1)
    rc = pkv::check_multi_query_step(q, k_pool, v_pool, page_table, context_lens, q_tokens, scale,
                                     workspace, workspace_bytes, groups ? ws.bytes : 0, out,
                                     lse_out, user_shape, shape, msg);
  else
    rc = pkv::check_step(q, k_new, v_new, k_pool, v_pool, page_table, context_lens, scale,
                         workspace, workspace_bytes, groups ? ws.bytes : 0, out, lse_out, shape,
                         msg);
  if (!rc && rope_cos)
    rc = pkv::check_rope_tables(k_new, rope_cos, rope_sin, rope_positions, out, lse_out, workspace,
                                workspace_bytes, shape, msg);
  if (rc) return set_error(rc, std::string(name) + ": " + msg);
  if (shape->batch == 0) return PKV_OK;
  pkv::StepParams p{};
  p.a = decode_params(q, k_pool, v_pool, page_table, context_lens, scale, *shape);
  p.a.heads_per_wg = step_heads_per_workgroup(*shape);
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool_w = k_pool;
  p.v_pool_w = v_pool;
  char* w = static_cast<char*>(workspace);
  p.ws_out = reinterpret_cast<float*>(w + ws.out_off);
  p.ws_lse = reinterpret_cast<float*>(w + ws.lse_off);
  p.ws_count = reinterpret_cast<uint64_t*>(w + ws.count_off);
  p.generation = take_generation();
  p.out = out;
  p.lse_out = lse_out;
  p.groups = int32_t(groups);
  p.append = k_new ? 1 : 0;
  // Several waves per KV head split its query heads when every wave gets at least one.
  const int wph = pkv::decode_waves() / p.a.heads_per_wg;
  const int gw = (p.a.group + wph - 1) / wph;
  p.qsplit = wph > 1 && (wph - 1) * gw < p.a.group ? 1 : 0;
  p.rope_cos = rope_cos;
  p.rope_sin = rope_sin;
  p.rope_rows = rope_positions;
  p.q_tokens = q_tokens;
  (void)hipGetLastError();
  return launch_status(pkv::launch_step(p, shape->dtype, shape->head_dim,
                                        group_pad(p.qsplit ? gw : p.a.group),
                                        static_cast<hipStream_t>(stream)),
                       name);
}
}  // namespace

int pkv_paged_decode_multi_query_step(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* page_table, const int32_t* context_lens,
                                      int32_t num_query_tokens, float scale, void* workspace,
                                      size_t workspace_bytes, void* out, float* lse_out,
                                      const pkv_shape* shape, void* stream) {
  if (num_query_tokens < 1)
    return set_error(PKV_EINVAL, "pkv_paged_decode_multi_query_step: num_query_tokens must be >= 1");
  return decode_step("pkv_paged_decode_multi_query_step", q, nullptr, nullptr,
                     const_cast<void*>(k_pool), const_cast<void*>(v_pool), page_table,
                     context_lens, nullptr, nullptr, 0, scale, workspace, workspace_bytes, out,
                     lse_out, shape, stream, num_query_tokens);
}

size_t pkv_multi_query_step_workspace_bytes(const pkv_shape* shape, int32_t num_query_tokens) {
  std::string msg;
  if (pkv::check_shape(shape, msg) != PKV_OK || num_query_tokens < 1) return 0;
  const pkv_shape v = step_shape(*shape, num_query_tokens);
  const int64_t groups = step_groups(v);
  if (groups == 0) return 0;
  return size_t(pkv::step_workspace(v, groups, step_heads_per_workgroup(v)).bytes);
}

int pkv_paged_decode_step(const void* q, const void* k_new, const void* v_new, void* k_pool,
                          void* v_pool, const int32_t* page_table, const int32_t* context_lens,
                          float scale, void* workspace, size_t workspace_bytes, void* out,
                          float* lse_out, const pkv_shape* shape, void* stream) {
  return decode_step("pkv_paged_decode_step", q, k_new, v_new, k_pool, v_pool, page_table,
                     context_lens, nullptr, nullptr, 0, scale, workspace, workspace_bytes, out,
                     lse_out, shape, stream);
}

}  // extern "C"

// Scratch of pkv_paged_decode_step_noalloc: the step's workspace (arrival counters, piece partials)
// in a static device array, for callers that cannot allocate.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` only names the symbol; its device
// address is looked up once per device (scratch_on_device) and only that address is used.
constexpr size_t kStepScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kStepScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
  bool cleared = false;   // the zeroing launch has been enqueued
};
ScratchSlot g_scratch_slots[kMaxScratchDevices];
std::mutex g_scratch_clear;

// The device address of `scratch` on `dev` (the current device): looked up on first use.
hipError_t scratch_on_device(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot& s = g_scratch_slots[dev];
  std::call_once(s.once, [&] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  *ptr = s.ptr;
  return s.err;
}

}  // namespace

extern "C" {

int pkv_paged_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                  void* k_pool, void* v_pool, const int32_t* page_table,
                                  const int32_t* context_lens, float scale, void* out,
                                  float* lse_out, const pkv_shape* shape, void* stream) {
  const char* name = "pkv_paged_decode_step_noalloc";
  std::string msg;
  int rc = pkv::check_shape(shape, msg);
  if (rc) return set_error(rc, std::string(name) + ": " + msg);
  if (shape->batch == 0) return PKV_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_error(PKV_ELAUNCH, std::string(name) + ": no device");
  const int64_t groups = step_groups(*shape);
  const uint64_t need =
      groups ? pkv::step_workspace(*shape, groups, step_heads_per_workgroup(*shape)).bytes : 0;
  if (need > kStepScratchBytes)
    return set_error(PKV_EWORKSPACE, std::string(name) + ": this shape needs " + std::to_string(need) +
                                         " bytes of step workspace, more than the " +
                                         std::to_string(kStepScratchBytes) +
                                         "-byte static scratch; use pkv_paged_decode_step with a "
                                         "workspace of that size");
  void* ptr = nullptr;
  const hipError_t e = scratch_on_device(dev, &ptr);
  if (e != hipSuccess)
    return set_error(PKV_ELAUNCH, std::string(name) + ": device address of the scratch: " +
                                      hipGetErrorString(e));
  {
    // The arrival counters must start at zero: the scratch is cleared once per device, on the
    // first call's stream, ahead of that call (later calls leave the counters at zero).
    std::lock_guard<std::mutex> lock(g_scratch_clear);
    ScratchSlot& s = g_scratch_slots[dev];
    if (!s.cleared) {
      (void)hipGetLastError();
      const int r = launch_status(pkv::launch_zero(ptr, kStepScratchBytes, static_cast<hipStream_t>(stream)), name);
      if (r) return r;
      s.cleared = true;
    }
  }
  return decode_step(name, q, k_new, v_new, k_pool, v_pool, page_table, context_lens, nullptr,
                     nullptr, 0, scale, ptr, kStepScratchBytes, out, lse_out, shape, stream);
}

int pkv_paged_decode_step_rope(const void* q, const void* k_new, const void* v_new, void* k_pool,
                               void* v_pool, const int32_t* page_table,
                               const int32_t* context_lens, const float* rope_cos,
                               const float* rope_sin, int32_t rope_positions, float scale,
                               void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                               const pkv_shape* shape, void* stream) {
  if (!rope_cos || !rope_sin || !k_new || !v_new)
    return set_error(PKV_EINVAL, "pkv_paged_decode_step_rope: rope_cos, rope_sin, k_new and "
                                 "v_new must be non-NULL (the rotated key is appended)");
  return decode_step("pkv_paged_decode_step_rope", q, k_new, v_new, k_pool, v_pool, page_table,
                     context_lens, rope_cos, rope_sin, rope_positions, scale, workspace,
                     workspace_bytes, out, lse_out, shape, stream);
}

int pkv_lse_merge(const float* partial_out, const float* partial_lse,
                  const int32_t* context_lens, int32_t partition_tokens, int32_t max_partitions,
                  void* out, float* lse_out, const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_merge(partial_out, partial_lse, context_lens, partition_tokens,
                                  max_partitions, out, lse_out, shape, msg);
  if (rc) return set_error(rc, "pkv_lse_merge: " + msg);
  if (shape->batch == 0) return PKV_OK;
  pkv::MergeParams p{};
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.context_lens = context_lens;
  p.out = out;
  p.lse_out = lse_out;
  p.batch = shape->batch;
  p.hq = shape->num_q_heads;
  p.partition_tokens = partition_tokens;
  p.max_partitions = max_partitions;
  p.capacity = shape->max_pages_per_seq * shape->page_size;
  (void)hipGetLastError();
  return launch_status(pkv::launch_merge(p, shape->dtype, shape->head_dim,
                                         static_cast<hipStream_t>(stream)),
                       "pkv_lse_merge");
}

int pkv_paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* page_table, const int32_t* context_lens,
                        const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_append(k_new, v_new, k_pool, v_pool, page_table, context_lens, shape, msg);
  if (rc) return set_error(rc, "pkv_paged_kv_append: " + msg);
  if (shape->batch == 0) return PKV_OK;
  pkv::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.page_table = page_table;
  p.context_lens = context_lens;
  p.batch = shape->batch;
  p.num_pages = shape->num_pages;
  p.max_pages = shape->max_pages_per_seq;
  p.page_shift = log2_exact(shape->page_size);
  p.capacity = shape->max_pages_per_seq * shape->page_size;
  p.row_bytes = shape->num_kv_heads * shape->head_dim * pkv::elem_bytes(shape->dtype);
  p.page_stride = int64_t(shape->page_size) * p.row_bytes;
  (void)hipGetLastError();
  return launch_status(pkv::launch_append(p, static_cast<hipStream_t>(stream)),
                       "pkv_paged_kv_append");
}

int pkv_rope_kv_append(const void* q, const void* k_new, const void* v_new, void* k_pool,
                       void* v_pool, const int32_t* page_table, const int32_t* context_lens,
                       const float* rope_cos, const float* rope_sin, int32_t rope_positions,
                       void* q_out, const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_rope_append(q, k_new, v_new, k_pool, v_pool, page_table, context_lens,
                                        rope_cos, rope_sin, rope_positions, q_out, shape, msg);
  if (rc) return set_error(rc, "pkv_rope_kv_append: " + msg);
  if (shape->batch == 0) return PKV_OK;
  pkv::RopeParams p{};
  p.a.k_new = k_new;
  p.a.v_new = v_new;
  p.a.k_pool = k_pool;
  p.a.v_pool = v_pool;
  p.a.page_table = page_table;
  p.a.context_lens = context_lens;
  p.a.batch = shape->batch;
  p.a.num_pages = shape->num_pages;
  p.a.max_pages = shape->max_pages_per_seq;
  p.a.page_shift = log2_exact(shape->page_size);
  p.a.capacity = shape->max_pages_per_seq * shape->page_size;
  p.a.row_bytes = shape->num_kv_heads * shape->head_dim * pkv::elem_bytes(shape->dtype);
  p.a.page_stride = int64_t(shape->page_size) * p.a.row_bytes;
  p.q = q;
  p.q_out = q_out;
  p.rope_cos = rope_cos;
  p.rope_sin = rope_sin;
  p.rope_rows = rope_positions;
  p.hq = shape->num_q_heads;
  p.hkv = shape->num_kv_heads;
  (void)hipGetLastError();
  return launch_status(pkv::launch_rope_append(p, shape->dtype, shape->head_dim,
                                               static_cast<hipStream_t>(stream)),
                       "pkv_rope_kv_append");
}

int pkv_copy_pages(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                   const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_copy_pages(k_pool, v_pool, pairs, n_pairs, shape, msg);
  if (rc) return set_error(rc, "pkv_copy_pages: " + msg);
  pkv::CopyPagesParams p{};
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.pairs = pairs;
  p.n = n_pairs;
  p.num_pages = shape->num_pages;
  p.page_bytes = int64_t(shape->page_size) * shape->num_kv_heads * shape->head_dim *
                 pkv::elem_bytes(shape->dtype);
  (void)hipGetLastError();
  return launch_status(pkv::launch_copy_pages(p, static_cast<hipStream_t>(stream)), "pkv_copy_pages");
}

int pkv_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return set_error(PKV_EINVAL, "pkv_read_stream: src and sink must be non-NULL");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || bytes % 16 != 0)
    return set_error(PKV_EINVAL, "pkv_read_stream: src and bytes must be multiples of 16");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return set_error(PKV_ELAUNCH, "pkv_read_stream: no device");
  (void)hipGetLastError();
  // One 8-wave workgroup per compute unit, each wave with 16 KB of loads in flight.
  return launch_status(pkv::launch_read_stream(src, bytes, sink, cus,
                                               static_cast<hipStream_t>(stream)),
                       "pkv_read_stream");
}

int pkv_validate_metadata(const int32_t* page_table, const int32_t* context_lens,
                          int32_t extra_tokens, int32_t check_append_unique,
                          int32_t* device_status, const pkv_shape* shape, void* stream) {
  std::string msg;
  const int rc = pkv::check_validate(page_table, context_lens, extra_tokens, device_status, shape, msg);
  if (rc) return set_error(rc, "pkv_validate_metadata: " + msg);
  pkv::ValidateParams p{};
  p.page_table = page_table;
  p.context_lens = context_lens;
  p.device_status = device_status;
  p.batch = shape->batch;
  p.num_pages = shape->num_pages;
  p.max_pages = shape->max_pages_per_seq;
  p.page_size = shape->page_size;
  p.extra_tokens = extra_tokens;
  p.check_append_unique = check_append_unique ? 1 : 0;
  (void)hipGetLastError();
  return launch_status(pkv::launch_validate(p, static_cast<hipStream_t>(stream)),
                       "pkv_validate_metadata");
}

}  // extern "C"
