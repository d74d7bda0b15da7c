// Chain verification of speculative drafts against the target's samples (the
// verify step of the TokenSpeed Triton sampling backend page: one target
// sample per row of the speculative layout, then each request's draft chain
// checked against them).  Request b owns rows b * n .. b * n + n - 1;
// candidates[b, 0] is its last verified token and candidates[b, 1..] its
// drafts.  Draft i + 1 is accepted while every earlier draft was and it equals
// the target sample of row b * n + i.  Positions 0 .. accepted emit the target
// sample and their row index; every other position gets -1.  One thread per
// request: a few integer compares, bound by launch latency.
#include "launch.hpp"

namespace tss {

namespace {

__global__ void verify_chain_kernel(int32_t bs, int32_t n, const int32_t* __restrict__ cand,
                                    const int32_t* __restrict__ tgt, int32_t* __restrict__ pred,
                                    int32_t* __restrict__ aidx, int32_t* __restrict__ alen) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < bs;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t base = b * n;
    int32_t acc = 0;
    while (acc + 1 < n && cand[base + acc + 1] == tgt[base + acc]) ++acc;
    for (int32_t i = 0; i < n; ++i) {
      const bool emit = i <= acc;
      pred[base + i] = emit ? tgt[base + i] : -1;
      aidx[base + i] = emit ? (int32_t)(base + i) : -1;
    }
    alen[b] = acc;
  }
}

}  // namespace

hipError_t launch_verify_chain(int32_t bs, int32_t n, const int32_t* candidates,
                               const int32_t* target_sampled, int32_t* predicts,
                               int32_t* accept_index, int32_t* accept_length, hipStream_t stream) {
  if (bs <= 0) return hipSuccess;
  const int block = 256;
  const int64_t blocks = ((int64_t)bs + block - 1) / block;
  const int grid = (int)(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(verify_chain_kernel, dim3(grid), dim3(block), 0, stream, bs, n, candidates,
                     target_sampled, predicts, accept_index, accept_length);
  return hipGetLastError();
}

}  // namespace tss
