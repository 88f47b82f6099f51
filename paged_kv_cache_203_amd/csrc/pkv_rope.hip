// Fused rotary embedding + paged KV append for the decode step's new token (gfx950).
//
// Every sequence b with L = context_lens[b] >= 0 has one new token at position L.  One workgroup
// per sequence, in one launch:
//  * rotates the token's query (every query head) into q_out;
//  * rotates its key (every KV head) and writes it to slot L % page_size of page
//    page_table[b][L / page_size] of the K pool;
//  * copies its value to the same slot of the V pool.
// The rotation is the rotate-half form: pair i < D/2 of a head is (x[i], x[i + D/2]), turned by
// the angle whose cosine and sine are rope_cos[L][i], rope_sin[L][i], in float32 (rope_pair),
// then rounded to the element type.  A thread takes 16 bytes of x[i..] and the matching 16 bytes
// of x[i + D/2..], so both halves of every pair sit in one thread.
// Padding rows (L < 0) copy q to q_out and write nothing.  Rows whose position has no row in the
// rotary cache (L >= rope_rows), or whose slot lies past the page table (L >= capacity), get NaN
// in q_out and write nothing; a page id out of range skips the write.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

using namespace dev;

template <int DT, int D>
__global__ __launch_bounds__(256) void rope_append_kernel(const RopeParams p) {
  using V = Vec16<DT>;
  constexpr int E = elem_size<DT>();
  constexpr int W = V::N;                 // elements (pairs) per 16 bytes
  constexpr int NCH = (D / 2) / W;        // 16-byte chunks per half head
  const AppendParams& a = p.a;
  const int b = blockIdx.x;
  const int L = a.context_lens[b];
  const bool pad = L < 0;
  const bool pos_ok = !pad && L < p.rope_rows && L < a.capacity;
  int page = -1;
  if (pos_ok) {
    page = a.page_table[int64_t(b) * a.max_pages + (L >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) page = -1;
  }
  const float* cs = p.rope_cos + int64_t(pos_ok ? L : 0) * (D / 2);
  const float* sn = p.rope_sin + int64_t(pos_ok ? L : 0) * (D / 2);

  // Rotate chunk j (pairs j*W .. j*W + W - 1) of the head row at byte `src`, into `dst`.
  auto rotate = [&](const char* src, char* dst, int j) {
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + j * 16);
    const u32x4 w2 = *reinterpret_cast<const u32x4*>(src + (D / 2) * E + j * 16);
    u32x4 o1 = w1, o2 = w2;
    if (pos_ok) {
      float x1[W], x2[W], y1[W], y2[W];
      V::unpack(w1, x1);
      V::unpack(w2, x2);
#pragma unroll
      for (int i = 0; i < W; ++i) rope_pair(x1[i], x2[i], cs[j * W + i], sn[j * W + i], y1[i], y2[i]);
      o1 = V::pack(y1);
      o2 = V::pack(y2);
    } else if (!pad) {
      float nan[W];
#pragma unroll
      for (int i = 0; i < W; ++i) nan[i] = qnan();
      o1 = o2 = V::pack(nan);
    }
    *reinterpret_cast<u32x4*>(dst + j * 16) = o1;
    *reinterpret_cast<u32x4*>(dst + (D / 2) * E + j * 16) = o2;
  };

  const int64_t qrow0 = int64_t(b) * p.hq;
  for (int t = threadIdx.x; t < p.hq * NCH; t += blockDim.x) {
    const int64_t off = (qrow0 + t / NCH) * D * E;
    rotate(static_cast<const char*>(p.q) + off, static_cast<char*>(p.q_out) + off, t % NCH);
  }
  if (page < 0) return;
  const int64_t dst = int64_t(page) * a.page_stride +
                      int64_t(L & ((1 << a.page_shift) - 1)) * a.row_bytes;
  const int64_t src = int64_t(b) * a.row_bytes;
  for (int t = threadIdx.x; t < p.hkv * NCH; t += blockDim.x) {
    const int64_t off = int64_t(t / NCH) * D * E;
    rotate(static_cast<const char*>(a.k_new) + src + off,
           static_cast<char*>(a.k_pool) + dst + off, t % NCH);
  }
  for (int i = threadIdx.x; i < a.row_bytes / 16; i += blockDim.x)
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.v_pool) + dst + 16 * i) =
        *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_new) + src + 16 * i);
}

template <int DT>
hipError_t launch_rope_dt(const RopeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL((rope_append_kernel<DT, 64>), dim3(unsigned(p.a.batch)), dim3(256), 0, stream, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL((rope_append_kernel<DT, 128>), dim3(unsigned(p.a.batch)), dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_append(const RopeParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (p.a.batch == 0) return hipSuccess;
  switch (dtype) {
    case DT_F32: return launch_rope_dt<DT_F32>(p, head_dim, stream);
    case DT_BF16: return launch_rope_dt<DT_BF16>(p, head_dim, stream);
    case DT_F16: return launch_rope_dt<DT_F16>(p, head_dim, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
