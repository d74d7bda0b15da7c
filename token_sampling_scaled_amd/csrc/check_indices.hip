// Debug check of the index arrays a sampling call reads through: gather
// indices must name a row of the logits buffer and request indices a slot of
// the parameter arrays.  ts_sample and ts_log_probs dereference both without
// a guard (their values live on the device, where checking every row would
// cost each call), so a caller that does not trust them runs this first.  One
// thread per row; each wave ORs its findings into the error word with one
// atomic.
#include "device_common.hpp"
#include "launch.hpp"

namespace tss {

namespace {

__global__ void clear_word_kernel(uint32_t* word) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *word = 0u;
}

__global__ void check_indices_kernel(int32_t n, const int32_t* __restrict__ gather, int64_t rows,
                                     const int32_t* __restrict__ req, int32_t num_requests,
                                     uint32_t* word) {
  uint32_t bits = 0;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n;
       r += (int64_t)gridDim.x * blockDim.x) {
    if (gather) {
      const int32_t g = gather[r];
      if (g < 0 || (int64_t)g >= rows) bits |= kIndexGatherOut;
    }
    if (req) {
      const int32_t q = req[r];
      if (q < 0 || q >= num_requests) bits |= kIndexRequestOut;
    }
  }
  const uint32_t wave_bits = (__ballot((bits & kIndexGatherOut) != 0) ? kIndexGatherOut : 0u) |
                             (__ballot((bits & kIndexRequestOut) != 0) ? kIndexRequestOut : 0u);
  if ((threadIdx.x & (kWave - 1)) == 0 && wave_bits != 0) atomicOr(word, wave_bits);
}

}  // namespace

hipError_t launch_check_indices(int32_t n, const int32_t* gather, int64_t rows, const int32_t* req,
                                int32_t num_requests, uint32_t* word, hipStream_t stream) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(kWave), 0, stream, word);
  if (n > 0 && (gather != nullptr || req != nullptr)) {
    const int block = 256;
    const int64_t blocks = ((int64_t)n + block - 1) / block;
    const int grid = (int)(blocks < 1024 ? blocks : 1024);
    hipLaunchKernelGGL(check_indices_kernel, dim3(grid), dim3(block), 0, stream, n, gather, rows,
                       req, num_requests, word);
  }
  return hipGetLastError();
}

}  // namespace tss
