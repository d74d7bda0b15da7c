// Device helpers shared by the sampling kernels (gfx950, wave64).
//
// Order keys, the Philox4x32-10 counter-based generator, the integer -> Gumbel
// transform and wave / block reductions.  Nothing here is shared with the CPU
// oracle: both follow the same published definitions independently.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tss {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Order keys: unsigned integers whose order is the order of the logits, with
// NaN read as -inf and -0 as +0 (so equal logits have equal keys).  Keys of
// finite values and +inf are strictly above key(-inf).

struct KeyF32 {
  static constexpr int kBits = 32;
  static constexpr uint32_t kNegInf = 0x007FFFFFu;          // key of 0xFF800000
  __device__ __forceinline__ static uint32_t from_bits(uint32_t u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;     // NaN -> -inf
    if (u == 0x80000000u) u = 0u;                             // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
};

struct KeyBF16 {
  static constexpr int kBits = 16;
  static constexpr uint32_t kNegInf = 0x007Fu;              // key of 0xFF80
  __device__ __forceinline__ static uint32_t from_bits(uint32_t b) {
    if ((b & 0x7FFFu) > 0x7F80u) b = 0xFF80u;                 // NaN -> -inf
    if (b == 0x8000u) b = 0u;                                 // -0 -> +0
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  }
};

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11, section 3): each round multiplies counter words 0 and 2
// by fixed 32-bit constants, swaps and xors the halves with the key, and the
// key advances by the Weyl constants between rounds.

struct Philox4 {
  uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  Philox4 r;
  r.v[0] = c0;
  r.v[1] = c1;
  r.v[2] = c2;
  r.v[3] = c3;
  return r;
}

// Noise stream of one output row: key = 64-bit seed, counter = (j >> 2, row,
// offset lo, offset hi); vocabulary index j reads word (j & 3).
struct NoiseStream {
  uint32_t k0, k1, row, off_lo, off_hi;
  __device__ __forceinline__ Philox4 block(uint32_t j4) const {
    return philox4x32_10(j4, row, off_lo, off_hi, k0, k1);
  }
  __device__ __forceinline__ uint32_t word(uint32_t j) const {
    const Philox4 b = block(j >> 2);
    const uint32_t s = j & 3u;
    return s == 0 ? b.v[0] : s == 1 ? b.v[1] : s == 2 ? b.v[2] : b.v[3];
  }
};

// u = (floor(w / 2^9) + 1/2) * 2^-23 is exact in fp32 and lies in
// [2^-24, 1 - 2^-24]; E = -ln u, g = -ln E.  E is taken from the hardware
// base-2 logarithm (v_log_f32) without a log1p branch for u near 1: its error
// on -log2(u) stays relative over the whole range, u = 1 - 2^-24 included.
// The probe library evaluates this function for every one of the 2^23 values
// of u and a GPU test holds it to the fp64 transform within a stated bound.
__device__ __forceinline__ float uniform_from_word(uint32_t w) {
  return ((float)(w >> 9) + 0.5f) * 0x1p-23f;
}

__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const float e = -__log2f(uniform_from_word(w)) * 0.69314718055994531f;
  return -__logf(e);
}

// The same noise in base-2 units, for kernels that race s2 = x log2(e) / T:
// g2 = -log2(-log2 u) = (g + ln ln 2) / ln 2, so argmax (s2 + g2) is
// argmax (x / T + g) (scaled by log2(e) and shifted by a constant).
__device__ __forceinline__ float gumbel2_from_word(uint32_t w) {
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(uniform_from_word(w)));
}

// ---------------------------------------------------------------------------
// Wave / block reductions (blockDim.x a multiple of 64).

template <typename V>
__device__ __forceinline__ V wave_sum(V v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, kWave);
    v = o < v ? o : v;
  }
  return v;
}

// DPP wave operations (row shifts inside each row of 16 lanes, then the row
// broadcasts of lanes 15 and 31).  Inclusive prefix sums over the 64 lanes:
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}

__device__ __forceinline__ float wave_scan_f32(float v) {
  v += dpp_f<0x111, 0xF>(v);
  v += dpp_f<0x112, 0xF>(v);
  v += dpp_f<0x114, 0xF>(v);
  v += dpp_f<0x118, 0xF>(v);
  v += dpp_f<0x142, 0xA>(v);
  v += dpp_f<0x143, 0xC>(v);
  return v;
}

// Wave-wide max / min (the result in every lane: the last lane's value):
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ float wave_max_f32_dpp(float v) {
  constexpr int kNegInf = (int)0xFF800000u;
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x111, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x112, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x114, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x118, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// (score, index) pair: larger score wins, smaller index on equal scores.
struct ArgBest {
  float z;
  int32_t j;
};

__device__ __forceinline__ bool better(float za, int32_t ja, float zb, int32_t jb) {
  return za > zb || (za == zb && ja < jb);
}

__device__ __forceinline__ ArgBest wave_argbest(ArgBest a) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float oz = __shfl_xor(a.z, off, kWave);
    const int32_t oj = __shfl_xor(a.j, off, kWave);
    if (better(oz, oj, a.z, a.j)) {
      a.z = oz;
      a.j = oj;
    }
  }
  return a;
}

}  // namespace tss
