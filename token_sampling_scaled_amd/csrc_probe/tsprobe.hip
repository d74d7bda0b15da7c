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

// Rows of any length: `parts` workgroups per row, each streaming its share of
// the row's 16-byte vectors with a ring of 16 loads in flight per thread (a
// vector processed is replaced at once by the one 16 vectors further on).
template <bool NT>
__global__ __launch_bounds__(kB) void read_rows_ring_kernel(const char* data, int64_t row_stride,
                                                            int32_t nvec, int32_t parts,
                                                            uint32_t* out) {
  constexpr int R = 16;
  const int row_i = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const v4u* row = reinterpret_cast<const v4u*>(data + (int64_t)row_i * row_stride);
  const int32_t per = (nvec + parts - 1) / parts;
  const int32_t v0 = part * per;
  const int32_t v1 = v0 + per < nvec ? v0 + per : nvec;
  const int nt = blockDim.x;
  const int tid = threadIdx.x;
  uint32_t x = 0;
  if (v0 < v1) {
    v4u ring[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int32_t vi = v0 + tid + u * nt;
      const v4u* p = row + (vi < v1 ? vi : v1 - 1);
      ring[u] = NT ? __builtin_nontemporal_load(p) : *p;
    }
    for (int32_t b = v0 + tid; b < v1; b += R * nt) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int32_t vi = b + u * nt;
        if (vi < v1) x ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
        const int32_t vn = vi + R * nt;
        const v4u* p = row + (vn < v1 ? vn : v1 - 1);
        ring[u] = NT ? __builtin_nontemporal_load(p) : *p;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, tss::kWave);
  __shared__ uint32_t acc;
  if (tid == 0) acc = 0;
  __syncthreads();
  if ((tid & (tss::kWave - 1)) == 0) atomicXor(&acc, x);
  __syncthreads();
  if (tid == 0) atomicXor(&out[row_i], acc);
}

__global__ __launch_bounds__(kB) void empty_kernel() {}

__global__ __launch_bounds__(256) void gumbel_table_kernel(float* g, float* g2) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;   // grid covers exactly 2^23
  const uint32_t w = i << 9;
  g[i] = tss::gumbel_from_word(w);
  g2[i] = tss::gumbel2_from_word(w);
}

// Noise throughput: each thread draws per_thread Philox4x32-10 blocks with
// counter (i, global thread, 0x5EED, 0) under a fixed key; with G every word
// also goes through the base-2 Gumbel transform and the thread keeps the
// largest result, as the sampling kernels do.  Each thread stores what it
// kept (so nothing is left out by the compiler).
template <bool G>
__global__ __launch_bounds__(256) void noise_rate_kernel(int32_t per_thread, uint32_t* out) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  uint32_t x = 0;
  float best = -__builtin_inff();
  for (int32_t i = 0; i < per_thread; ++i) {
    const tss::Philox4 b = tss::philox4x32_10((uint32_t)i, t, 0x5EEDu, 0u, 0x9E3779B9u, 0x7F4A7C15u);
    if (G) {
#pragma unroll
      for (int e = 0; e < 4; ++e) best = fmaxf(best, tss::gumbel2_from_word(b.v[e]));
    } else {
      x ^= b.v[0] ^ b.v[1] ^ b.v[2] ^ b.v[3];
    }
  }
  out[t] = G ? __float_as_uint(best) : x;
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

int tsp_read_rows_ring(const void* data, int64_t rows, int64_t row_bytes, int64_t row_stride_bytes,
                       int32_t threads, int32_t parts, int32_t nontemporal, uint32_t* out,
                       void* stream) {
  if (data == nullptr || out == nullptr || rows < 1 || row_bytes < 16 || (row_bytes % 16) != 0 ||
      (row_stride_bytes % 16) != 0 || row_stride_bytes < row_bytes || row_bytes / 16 > 0x7FFFFFFF ||
      (reinterpret_cast<uintptr_t>(data) % 16) != 0 ||
      (threads != 256 && threads != 512 && threads != 1024) || parts < 1 || parts > 64 ||
      rows * parts > 0x7FFFFFFF)
    return 1;
  const dim3 grid((uint32_t)(rows * parts)), block((uint32_t)threads);
  const char* d = static_cast<const char*>(data);
  const int32_t nvec = (int32_t)(row_bytes / 16);
  if (nontemporal)
    hipLaunchKernelGGL(read_rows_ring_kernel<true>, grid, block, 0, (hipStream_t)stream, d,
                       row_stride_bytes, nvec, parts, out);
  else
    hipLaunchKernelGGL(read_rows_ring_kernel<false>, grid, block, 0, (hipStream_t)stream, d,
                       row_stride_bytes, nvec, parts, out);
  return launched();
}

int tsp_empty(int32_t blocks, void* stream) {
  if (blocks < 1) return 1;
  hipLaunchKernelGGL(empty_kernel, dim3((uint32_t)blocks), dim3(kB), 0, (hipStream_t)stream);
  return launched();
}

int tsp_noise_rate(int32_t blocks, int32_t per_thread, int32_t with_gumbel, uint32_t* out,
                   void* stream) {
  if (out == nullptr || blocks < 1 || per_thread < 1 || (int64_t)blocks * 256 > 0x7FFFFFFF) return 1;
  if (with_gumbel)
    hipLaunchKernelGGL(noise_rate_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0,
                       (hipStream_t)stream, per_thread, out);
  else
    hipLaunchKernelGGL(noise_rate_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0,
                       (hipStream_t)stream, per_thread, out);
  return launched();
}

int tsp_gumbel_table(float* g, float* g2, void* stream) {
  if (g == nullptr || g2 == nullptr) return 1;
  hipLaunchKernelGGL(gumbel_table_kernel, dim3((1u << 23) / 256u), dim3(256), 0,
                     (hipStream_t)stream, g, g2);
  return launched();
}

}  // extern "C"
