// Launch of multi-query decode on the matrix cores (the prefix kernel body in its per-sequence
// mode; the body and its design are in pkv_prefix_body.h, and the shared-prefix partitions run it
// inside cascade_kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_prefix_body.h"

namespace pkv {
namespace {

using namespace dev;

template <int DT, int D, int NW, int RBW, bool MQ>
__global__ __launch_bounds__(NW * 64) void prefix_kernel(const PrefixParams p) {
  __shared__ PrefixShared<D> sm;
  prefix_body<DT, D, NW, RBW, MQ>(p, blockIdx.x, sm);
}

template <int DT, int D, int NW>
hipError_t launch_multi_query_t(const PrefixParams& p, hipStream_t stream) {
  constexpr int ROWS = PrefixGeo<D, NW, 1>::ROWS;
  const int64_t tiles = (int64_t(p.q_tokens) * p.group + ROWS - 1) / ROWS;
  const int64_t units = tiles * p.max_partitions * p.batch * p.hkv;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((prefix_kernel<DT, D, NW, 1, true>), dim3(unsigned(units)), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_prefix_t(const PrefixParams& p, hipStream_t stream) {
  // (row tile, partition, sequence, KV head).  Up to 64 rows (G x T): 4-wave workgroups, two per
  // compute unit, so that two blocks of K/V are in flight per unit; more rows: 8-wave workgroups
  // of 128 rows.
  if (int64_t(p.q_tokens) * p.group <= 64) return launch_multi_query_t<DT, D, 4>(p, stream);
  return launch_multi_query_t<DT, D, 8>(p, stream);
}

}  // namespace

hipError_t launch_prefix(const PrefixParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (p.q_tokens <= 0) return hipErrorInvalidValue;   // the shared prefix runs in cascade_kernel
  if (p.batch == 0) return hipSuccess;
  switch (dtype) {
    case DT_BF16:
      return head_dim == 64 ? launch_prefix_t<DT_BF16, 64>(p, stream)
                            : launch_prefix_t<DT_BF16, 128>(p, stream);
    case DT_F16:
      return head_dim == 64 ? launch_prefix_t<DT_F16, 64>(p, stream)
                            : launch_prefix_t<DT_F16, 128>(p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pkv
