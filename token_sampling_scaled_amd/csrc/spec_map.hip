// Request index of each row in the speculative-verify layout
// ("core.inference.sampling.base", sample_speculative): decode request d owns
// 1 + num_spec consecutive rows starting at d * (1 + num_spec); prefill request
// i owns the single row num_decode * (1 + num_spec) + i and has index
// num_decode + i.
#include "launch.hpp"

namespace tss {

namespace {

__global__ void spec_map_kernel(int32_t num_decode, int32_t num_prefill, int32_t num_spec,
                                int32_t* out_map) {
  const int64_t per = 1 + (int64_t)num_spec;
  const int64_t decode_rows = (int64_t)num_decode * per;
  const int64_t n = decode_rows + num_prefill;
  for (int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; row < n;
       row += (int64_t)gridDim.x * blockDim.x)
    out_map[row] = row < decode_rows ? (int32_t)(row / per)
                                     : (int32_t)(num_decode + (row - decode_rows));
}

}  // namespace

hipError_t launch_spec_map(int32_t num_decode, int32_t num_prefill, int32_t num_spec,
                           int32_t* out_map, hipStream_t stream) {
  const int64_t n = (int64_t)num_decode * (1 + (int64_t)num_spec) + num_prefill;
  if (n <= 0) return hipSuccess;
  const int block = 256;
  const int64_t blocks = (n + block - 1) / block;
  const int grid = (int)(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(spec_map_kernel, dim3(grid), dim3(block), 0, stream, num_decode,
                     num_prefill, num_spec, out_map);
  return hipGetLastError();
}

}  // namespace tss
