// Measurement probes (libtsprobe.so): a plain streaming read with the launch
// shape of the register-resident sampling kernel, an empty launch, and the
// device noise transforms over their whole input domain.  See
// include/tsprobe.h for the contract of each entry point.
#include "tsprobe.h"

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace {

constexpr int kB = 1024;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// One workgroup per row; thread t reads vectors t, t + 1024, ... (all loads
// issued before the first use), exactly the order of the sampling kernel.
// Slots past the row re-read its last vector (every load stays in bounds) and
// are left out of the xor, so out[row] is the xor of each vector once.
template <int NV>
__global__ __launch_bounds__(kB) void read_rows_kernel(const char* data, int64_t row_stride,
                                                       int32_t nvec, uint32_t* out) {
  const v4u* row = reinterpret_cast<const v4u*>(data + (int64_t)blockIdx.x * row_stride);
  const int tid = threadIdx.x;
  v4u d[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = i * kB + tid;
    d[i] = __builtin_nontemporal_load(row + (vi < nvec ? vi : nvec - 1));
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (i * kB + tid < nvec) x ^= d[i].x ^ d[i].y ^ d[i].z ^ d[i].w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, tss::kWave);
  __shared__ uint32_t acc;
  if (tid == 0) acc = 0;
  __syncthreads();
  if ((tid & (tss::kWave - 1)) == 0) atomicXor(&acc, x);
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kB) void empty_kernel() {}

__global__ __launch_bounds__(256) void gumbel_table_kernel(float* g, float* g2) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;   // grid covers exactly 2^23
  const uint32_t w = i << 9;
  g[i] = tss::gumbel_from_word(w);
  g2[i] = tss::gumbel2_from_word(w);
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : 4; }

}  // namespace

extern "C" {

int tsp_read_rows(const void* data, int64_t rows, int64_t row_bytes, int64_t row_stride_bytes,
                  int32_t loads_per_thread, uint32_t* out, void* stream) {
  if (data == nullptr || out == nullptr || rows < 1 || rows > 0x7FFFFFFF || row_bytes < 16 ||
      (row_bytes % 16) != 0 || (row_stride_bytes % 16) != 0 || row_stride_bytes < row_bytes ||
      (reinterpret_cast<uintptr_t>(data) % 16) != 0)
    return 1;
  const int64_t nvec = row_bytes / 16;
  const int nv = loads_per_thread;
  if ((nv != 1 && nv != 2 && nv != 4 && nv != 8 && nv != 16) || nvec > (int64_t)nv * kB) return 1;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid((uint32_t)rows), block(kB);
  const char* d = static_cast<const char*>(data);
  switch (nv) {
    case 1: hipLaunchKernelGGL(read_rows_kernel<1>, grid, block, 0, s, d, row_stride_bytes, (int32_t)nvec, out); break;
    case 2: hipLaunchKernelGGL(read_rows_kernel<2>, grid, block, 0, s, d, row_stride_bytes, (int32_t)nvec, out); break;
    case 4: hipLaunchKernelGGL(read_rows_kernel<4>, grid, block, 0, s, d, row_stride_bytes, (int32_t)nvec, out); break;
    case 8: hipLaunchKernelGGL(read_rows_kernel<8>, grid, block, 0, s, d, row_stride_bytes, (int32_t)nvec, out); break;
    default: hipLaunchKernelGGL(read_rows_kernel<16>, grid, block, 0, s, d, row_stride_bytes, (int32_t)nvec, out); break;
  }
  return launched();
}

int tsp_empty(int32_t blocks, void* stream) {
  if (blocks < 1) return 1;
  hipLaunchKernelGGL(empty_kernel, dim3((uint32_t)blocks), dim3(kB), 0, (hipStream_t)stream);
  return launched();
}

int tsp_gumbel_table(float* g, float* g2, void* stream) {
  if (g == nullptr || g2 == nullptr) return 1;
  hipLaunchKernelGGL(gumbel_table_kernel, dim3((1u << 23) / 256u), dim3(256), 0,
                     (hipStream_t)stream, g, g2);
  return launched();
}

}  // extern "C"
