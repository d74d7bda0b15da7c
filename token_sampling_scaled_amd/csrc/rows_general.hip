// General row kernel: one workgroup of 1024 threads per output row running
// the general per-row body (see general_row.hpp).
#include "general_row.hpp"

namespace tss {

namespace {

using general::kBlock;
using general::Shared;

template <typename T, int ROUTE, int MODE>
__global__ __launch_bounds__(kBlock) void rows_general_kernel(RowArgs a) {
  __shared__ Shared sh;
  general::general_row<T, ROUTE, MODE>(a, blockIdx.x, sh);
}

template <typename T, int ROUTE>
hipError_t launch_mode(const RowArgs& a, OutMode mode, hipStream_t stream) {
  const dim3 grid(a.n), block(kBlock);
  switch (mode) {
    case kOutSample:
      hipLaunchKernelGGL((rows_general_kernel<T, ROUTE, kOutSample>), grid, block, 0, stream, a);
      break;
    case kOutLogProbFull:
      hipLaunchKernelGGL((rows_general_kernel<T, ROUTE, kOutLogProbFull>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((rows_general_kernel<T, ROUTE, kOutLogProbAt>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_route(const RowArgs& a, Route route, OutMode mode, hipStream_t stream) {
  switch (route) {
    case kRouteNone: return launch_mode<T, kRouteNone>(a, mode, stream);
    case kRouteTopK: return launch_mode<T, kRouteTopK>(a, mode, stream);
    case kRouteTopP: return launch_mode<T, kRouteTopP>(a, mode, stream);
    default: return launch_mode<T, kRouteJoint>(a, mode, stream);
  }
}

}  // namespace

hipError_t launch_rows_general(const RowArgs& a, DType dtype, Route route, OutMode mode,
                               hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  return dtype == kF32 ? launch_route<float>(a, route, mode, stream)
                       : launch_route<uint16_t>(a, route, mode, stream);
}

}  // namespace tss
