// Plain read stream of device memory (gfx950): the achievable HBM read rate on this device, the
// ceiling that the decode kernels' algorithmic bytes per second are compared with beside the
// published peak.  Every byte of the buffer is read once with 16-byte non-temporal loads (the
// policy the decode kernels stream K and V rows with); the words are folded by XOR so that no
// load is dead, and each workgroup folds its value into one word of `sink`.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per thread

__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const char* base, uint64_t chunks,
                                                                     uint32_t* sink) {
  const gptr src = to_gptr(base);
  const uint64_t stride = uint64_t(gridDim.x) * kStreamThreads;
  uint64_t i = uint64_t(blockIdx.x) * kStreamThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kStreamUnroll - 1) * stride < chunks; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = stream_load16(src + (i + u * stride) * 16);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  for (; i < chunks; i += stride) acc ^= stream_load16(src + i * 16);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0 && x != 0) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_read_stream(const void* src, uint64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(workgroups)), dim3(kStreamThreads), 0,
                     stream, static_cast<const char*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
