// Device helpers of the split-row kernels (rows spread over several
// workgroups): entry loading in 4-entry groups (one Philox block each), the
// (max, sum) log-sum-exp pair, the order word of a best entry, and
// device-coherent stores and loads for the partial results.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace tss {
namespace split {

constexpr int kSplitBlock = 256;
constexpr int kSplitWaves = kSplitBlock / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct SplitElem;

template <>
struct SplitElem<float> {
  using Key = KeyF32;
  using Packed = u32x4;
  static constexpr uint32_t kNegInfRaw = 0xFF800000u;
  __device__ __forceinline__ static float value(uint32_t raw) { return __uint_as_float(raw); }
  __device__ __forceinline__ static uint32_t raw_at(const void* row, int64_t j) {
    return __float_as_uint(static_cast<const float*>(row)[j]);
  }
  // Entries j0 .. j0+3, present and 16-byte aligned.
  __device__ __forceinline__ static Packed load_packed(const void* row, int64_t j0) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        reinterpret_cast<const float*>(row) + j0));
  }
  __device__ __forceinline__ static void unpack(const Packed& q, uint32_t raw[4]) {
    raw[0] = q.x;
    raw[1] = q.y;
    raw[2] = q.z;
    raw[3] = q.w;
  }
  // Entries j0 .. j0+3 one by one (past the row: -inf).
  __device__ __forceinline__ static void load4(const void* row, int64_t j0, int64_t v,
                                               uint32_t raw[4]) {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = (j0 + i < v) ? u[j0 + i] : kNegInfRaw;
  }
};

template <>
struct SplitElem<uint16_t> {
  using Key = KeyBF16;
  using Packed = u32x2;
  static constexpr uint32_t kNegInfRaw = 0xFF80u;
  __device__ __forceinline__ static float value(uint32_t raw) { return __uint_as_float(raw << 16); }
  __device__ __forceinline__ static uint32_t raw_at(const void* row, int64_t j) {
    return static_cast<const uint16_t*>(row)[j];
  }
  __device__ __forceinline__ static Packed load_packed(const void* row, int64_t j0) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
        reinterpret_cast<const uint16_t*>(row) + j0));
  }
  __device__ __forceinline__ static void unpack(const Packed& q, uint32_t raw[4]) {
    raw[0] = q.x & 0xFFFFu;
    raw[1] = q.x >> 16;
    raw[2] = q.y & 0xFFFFu;
    raw[3] = q.y >> 16;
  }
  __device__ __forceinline__ static void load4(const void* row, int64_t j0, int64_t v,
                                               uint32_t raw[4]) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = (j0 + i < v) ? (uint32_t)p[j0 + i] : kNegInfRaw;
  }
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)v, off, kWave);
    if ((threadIdx.x & (kWave - 1)) >= (unsigned)off) v += o;
  }
  return v;
}

// (max, sum) pair of a base-2 log-sum-exp: sum of exp2(s - max) over the
// entries seen.
struct Lse {
  float m;
  float sum;
};

__device__ __forceinline__ Lse lse_merge(Lse a, Lse b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -__builtin_inff()) return Lse{m, 0.0f};
  return Lse{m, a.sum * __builtin_amdgcn_exp2f(a.m - m) + b.sum * __builtin_amdgcn_exp2f(b.m - m)};
}

__device__ __forceinline__ Lse wave_lse(Lse v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Lse o{__shfl_xor(v.m, off, kWave), __shfl_xor(v.sum, off, kWave)};
    v = lse_merge(v, o);
  }
  return v;
}

// Best entry so far: o is an unsigned order word (the perturbed score made
// order-preserving, or the logit's order key for greedy rows; 0 = none), ties
// go to the smaller index; s is the winner's scaled logit (base 2).
struct Best {
  uint32_t o;
  int32_t j;
  float s;
};

__device__ __forceinline__ uint32_t order_of(float z) {
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool beats(uint32_t oa, int32_t ja, uint32_t ob, int32_t jb) {
  return oa > ob || (oa == ob && ja < jb);
}

__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Best o{(uint32_t)__shfl_xor((int)b.o, off, kWave), __shfl_xor(b.j, off, kWave),
                 __shfl_xor(b.s, off, kWave)};
    if (beats(o.o, o.j, b.o, b.j)) b = o;
  }
  return b;
}

__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent_f(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int32_t load_agent_i(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent_u(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace split
}  // namespace tss
