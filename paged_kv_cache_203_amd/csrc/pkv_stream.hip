// Plain read stream of device memory (gfx950): the achievable HBM read rate on this device, the
// ceiling that the decode kernels' algorithmic bytes per second are compared with beside the
// published peak.  Every byte of the buffer is read once with the loads the decode kernels stream
// K rows with: 16-byte direct-to-LDS loads (non-temporal), so that the data never occupies
// registers and each wave keeps kStreamDepth loads in flight.  One workgroup per compute unit.
// What lands in LDS is discarded, except one word per workgroup folded into *sink (XOR).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kStreamWaves = 8;
constexpr int kStreamDepth = 16;   // 1 KB direct-to-LDS loads in flight per wave

__global__ __launch_bounds__(kStreamWaves * 64) void read_stream_kernel(const char* base,
                                                                       uint64_t chunks,
                                                                       uint32_t* sink) {
  __shared__ char land[kStreamWaves][kStreamDepth][1024] __attribute__((aligned(16)));
  const gptr src = to_gptr(base);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // Chunks of 64 x 16 bytes (one load instruction of a wave), dealt to the waves round-robin.
  const uint64_t waves = uint64_t(gridDim.x) * kStreamWaves;
  const uint64_t blocks = chunks / 64;
  uint64_t j = uint64_t(blockIdx.x) * kStreamWaves + wave;
  const uint32_t dst0 = lds_addr(&land[wave][0][0]);
  int slot = 0;
  for (; j < blocks; j += waves) {
    dma16_to_lds<kDmaPolicy>(src + (j * 64 + lane) * 16, dst0 + uint32_t(slot) * 1024u);
    slot = slot + 1 == kStreamDepth ? 0 : slot + 1;
    // at most kStreamDepth loads in flight: the slot about to be reused has landed
    wait_vmcnt<kStreamDepth - 1>();
  }
  // the remaining chunks (fewer than 64 of 16 bytes) go through wave 0 of workgroup 0
  if (blockIdx.x == 0 && wave == 0) {
    const uint64_t i = blocks * 64 + lane;
    if (i < chunks) dma16_to_lds<kDmaPolicy>(src + i * 16, dst0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(&land[0][0][0]);
    if (x != 0) atomicXor(sink, x);
  }
}

}  // namespace

hipError_t launch_read_stream(const void* src, uint64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(workgroups)), dim3(kStreamWaves * 64), 0,
                     stream, static_cast<const char*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
