// Per-row body of the general sampling path (one workgroup of 1024 threads per
// row, any vocabulary size, dtype, k and p).  Each step is a pass over the row
// in global memory (re-reads hit L2 / the Infinity Cache):
//
//   A  max key, its lowest index and the finite count  (one pass)
//   K  top-k threshold: radix select on order keys, 8 bits per pass, then the
//      lowest-index members of the boundary tie group by a radix select on the
//      inverted index                                  (only rows with top-k)
//   P  top-p cutoff: the largest key v with mass(key >= v) >= p * mass(K).
//      With k <= 1024, from K's members gathered in shared memory (each
//      member's mass above it); otherwise a radix select on probability mass,
//      8 bits per pass                                   (only rows with top-p)
//   F  Philox noise and the perturbed argmax over P, plus the mass of P
//
// Probability masses are summed as 64-bit fixed-point integers, so every sum is
// independent of the order of the atomics and the result is bitwise
// reproducible.  The fast kernels fall back to this body for rows they do not
// cover.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace tss {


namespace general {

constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / kWave;

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  using Key = KeyF32;
  static constexpr uint32_t kNegInfRaw = 0xFF800000u;
  __device__ __forceinline__ static float value(uint32_t raw) { return __uint_as_float(raw); }
  __device__ __forceinline__ static uint32_t key_to_raw(uint32_t k) {
    return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  }
  __device__ __forceinline__ static void load4(const float* row, int64_t j0, int64_t v, bool vec,
                                               uint32_t raw[4]) {
    if (vec && j0 + 4 <= v) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + j0);
      raw[0] = q.x;
      raw[1] = q.y;
      raw[2] = q.z;
      raw[3] = q.w;
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = (j0 + i < v) ? p[j0 + i] : kNegInfRaw;
    }
  }
};

template <>
struct Elem<uint16_t> {
  using Key = KeyBF16;
  static constexpr uint32_t kNegInfRaw = 0xFF80u;
  __device__ __forceinline__ static float value(uint32_t raw) { return __uint_as_float(raw << 16); }
  __device__ __forceinline__ static uint32_t key_to_raw(uint32_t k) {
    return (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  }
  __device__ __forceinline__ static void load4(const uint16_t* row, int64_t j0, int64_t v, bool vec,
                                               uint32_t raw[4]) {
    if (vec && j0 + 4 <= v) {
      const uint2 q = *reinterpret_cast<const uint2*>(row + j0);
      raw[0] = q.x & 0xFFFFu;
      raw[1] = q.x >> 16;
      raw[2] = q.y & 0xFFFFu;
      raw[3] = q.y >> 16;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = (j0 + i < v) ? (uint32_t)row[j0 + i] : kNegInfRaw;
    }
  }
};

// Calls f(j0, raw[4]) for the groups of four consecutive entries this thread owns.
template <typename T, typename F>
__device__ __forceinline__ void for_groups(const T* row, int64_t v, bool vec, F&& f) {
  const int64_t groups = (v + 3) >> 2;
  for (int64_t g = threadIdx.x; g < groups; g += kBlock) {
    uint32_t raw[4];
    Elem<T>::load4(row, g << 2, v, vec, raw);
    f(g << 2, raw);
  }
}

// Radix step: the largest digit d with reach(base + S(d)), S(d) = sum of
// hist[d'] over d' >= d.  Every wave evaluates it on its own (no barrier).
// *above = base + S(d + 1), *bin = hist[d].
template <typename C, typename Reach>
__device__ __forceinline__ int find_digit_desc(const C* hist, C base, Reach reach, C* above, C* bin) {
  const int lane = threadIdx.x & (kWave - 1);
  C h[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) h[b] = hist[4 * lane + b];
  C t = h[0] + h[1] + h[2] + h[3];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const C o = __shfl_down(t, off, kWave);
    if (lane + off < kWave) t += o;
  }
  const unsigned long long m = __ballot(reach(base + t));
  const int top = m ? 63 - __clzll((long long)m) : 0;
  C next = __shfl(t, (top + 1) & (kWave - 1), kWave);
  if (top == kWave - 1) next = 0;
  C acc = base + next;
  int d = 4 * top;
  C hb = hist[4 * top];
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    const C hv = hist[4 * top + b];
    if (reach(acc + hv)) {
      d = 4 * top + b;
      hb = hv;
      break;
    }
    acc += hv;
  }
  *above = acc;
  *bin = hb;
  return d;
}

// Largest top-k whose members are gathered in shared memory for the top-p
// cutoff (K has exactly k entries).
constexpr int kKMax = 1024;

struct Shared {
  uint32_t hist32[256];
  unsigned long long hist64[256];
  uint32_t wkey[kWaves];
  int32_t widx[kWaves];
  unsigned long long wsum[kWaves];
  float wz[kWaves];
  alignas(16) uint32_t kkey[kKMax];              // members of K: order keys ...
  alignas(16) unsigned long long kmass[kKMax];   // ... and fixed-point masses
  uint32_t nk;
  uint32_t vcmin;
};

__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, Shared& sh) {
  v = wave_sum(v);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sh.wsum[wid] = v;
  __syncthreads();
  unsigned long long t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += sh.wsum[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ ArgBest block_argbest(ArgBest a, Shared& sh) {
  a = wave_argbest(a);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.wz[wid] = a.z;
    sh.widx[wid] = a.j;
  }
  __syncthreads();
  ArgBest b{sh.wz[0], sh.widx[0]};
#pragma unroll
  for (int w = 1; w < kWaves; ++w)
    if (better(sh.wz[w], sh.widx[w], b.z, b.j)) b = ArgBest{sh.wz[w], sh.widx[w]};
  __syncthreads();
  return b;
}

template <typename T, int ROUTE, int MODE>
__device__ __forceinline__ void general_row(const RowArgs& a, int r, Shared& sh) {
  using E = Elem<T>;
  using Key = typename E::Key;
  constexpr bool kHasK = (ROUTE == kRouteTopK || ROUTE == kRouteJoint);
  constexpr bool kHasP = (ROUTE == kRouteTopP || ROUTE == kRouteJoint);
  const int tid = threadIdx.x;
  const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
  const int64_t q = a.req_map ? (int64_t)a.req_map[r] : (int64_t)r;
  const T* row = reinterpret_cast<const T*>(a.logits) + src * a.row_stride;
  const int64_t v = a.vocab;
  const bool vec = (reinterpret_cast<uintptr_t>(row) % (4 * sizeof(T))) == 0;
  const float temp = a.temperature[q];
  const int32_t kq = kHasK ? a.top_k[q] : 0;
  const float pq = kHasP ? a.top_p[q] : 1.0f;

  // ---- A: max key (lowest index among equal keys) and finite count.
  uint32_t bkey = 0;
  int32_t bidx = 0x7FFFFFFF;
  uint32_t nfin = 0;
  for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t k = Key::from_bits(raw[i]);
      const int32_t j = (int32_t)(j0 + i);
      nfin += (k > Key::kNegInf) ? 1u : 0u;
      if (k > bkey || (k == bkey && j < bidx)) {
        bkey = k;
        bidx = j;
      }
    }
  });
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t ok = __shfl_xor(bkey, off, kWave);
    const int32_t oj = __shfl_xor(bidx, off, kWave);
    if (ok > bkey || (ok == bkey && oj < bidx)) {
      bkey = ok;
      bidx = oj;
    }
  }
  nfin = wave_sum(nfin);
  if ((tid & (kWave - 1)) == 0) {
    sh.wkey[tid / kWave] = bkey;
    sh.widx[tid / kWave] = bidx;
    sh.wsum[tid / kWave] = nfin;
  }
  __syncthreads();
  uint32_t kmax = 0;
  int32_t jmax = 0x7FFFFFFF;
  uint32_t nfinite = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t k = sh.wkey[w];
    if (k > kmax || (k == kmax && sh.widx[w] < jmax)) {
      kmax = k;
      jmax = sh.widx[w];
    }
    nfinite += (uint32_t)sh.wsum[w];
  }
  __syncthreads();

  // ---- rows with no finite logit, greedy rows
  if (nfinite == 0) {
    if (MODE == kOutSample) {
      if (tid == 0) {
        a.out_ids[r] = -1;
        if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
      }
    } else if (MODE == kOutLogProbAt) {
      if (tid == 0) a.out_lp[r] = __builtin_nanf("");
    } else {
      for (int64_t j = tid; j < v; j += kBlock) a.out_lp[r * v + j] = __builtin_nanf("");
    }
    return;
  }
  if (!(temp >= 1e-5f)) {
    if (MODE == kOutSample) {
      if (tid == 0) {
        a.out_ids[r] = jmax;
        if (a.out_lp) a.out_lp[r] = 0.0f;
      }
    } else if (MODE == kOutLogProbAt) {
      if (tid == 0) a.out_lp[r] = (a.token_ids[r] == jmax) ? 0.0f : -__builtin_inff();
    } else {
      for (int64_t j = tid; j < v; j += kBlock)
        a.out_lp[r * v + j] = (j == jmax) ? 0.0f : -__builtin_inff();
    }
    return;
  }

  const float inv_t = 1.0f / temp;
  const float m = __fmul_rn(E::value(E::key_to_raw(kmax)), inv_t);
  const float scale = __builtin_ldexpf(1.0f, a.mass_shift);

  // ---- K: top-k threshold (tau) and the last admitted index of its tie group.
  const bool k_on = kHasK && kq >= 1 && (int64_t)kq < v && (uint32_t)kq < nfinite;
  uint32_t tau = 0;
  int64_t idx_cut = v;
  if (k_on) {
    uint32_t prefix = 0, pmask = 0, above = 0, bin = 0;
    const uint32_t need = (uint32_t)kq;
    for (int shift = Key::kBits - 8; shift >= 0; shift -= 8) {
      if (tid < 256) sh.hist32[tid] = 0;
      __syncthreads();
      for_groups(row, v, vec, [&](int64_t, const uint32_t* raw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t k = Key::from_bits(raw[i]);
          if (k > Key::kNegInf && (k & pmask) == prefix) atomicAdd(&sh.hist32[(k >> shift) & 255u], 1u);
        }
      });
      __syncthreads();
      const int d = find_digit_desc<uint32_t>(sh.hist32, above,
                                              [&](uint32_t c) { return c >= need; }, &above, &bin);
      prefix |= (uint32_t)d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    tau = prefix;
    const uint32_t ties_needed = need - above;
    if (ties_needed < bin) {
      // Smallest `ties_needed` indices among key == tau: the largest inverted indices.
      const uint32_t top_idx = (a.index_bits >= 32) ? 0xFFFFFFFFu : ((1u << a.index_bits) - 1u);
      uint32_t ip = 0, im = 0, iabove = 0, ibin = 0;
      const int first_shift = ((a.index_bits + 7) / 8) * 8 - 8;
      for (int shift = first_shift; shift >= 0; shift -= 8) {
        if (tid < 256) sh.hist32[tid] = 0;
        __syncthreads();
        for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k = Key::from_bits(raw[i]);
            const uint32_t inv = top_idx - (uint32_t)(j0 + i);
            if (k == tau && (inv & im) == ip) atomicAdd(&sh.hist32[(inv >> shift) & 255u], 1u);
          }
        });
        __syncthreads();
        const int d = find_digit_desc<uint32_t>(
            sh.hist32, iabove, [&](uint32_t c) { return c >= ties_needed; }, &iabove, &ibin);
        ip |= (uint32_t)d << shift;
        im |= 255u << shift;
        __syncthreads();
      }
      idx_cut = (int64_t)(top_idx - ip);
    }
  }
  auto in_k = [&](uint32_t k, int64_t j) -> bool {
    return k > Key::kNegInf && (!k_on || k > tau || (k == tau && j <= idx_cut));
  };
  auto fixed_mass = [&](uint32_t raw) -> unsigned long long {
    const float w = __expf(__fmaf_rn(E::value(raw), inv_t, -m));
    return __float2ull_rn(w * scale);
  };

  // ---- P: top-p cutoff key vc (P = K and key >= vc).
  const bool p_on = kHasP && pq < 1.0f - 1e-6f;
  uint32_t vc = 0;
  if (p_on) {
    if (!(pq > 0.0f)) {
      vc = kmax;
    } else if (k_on && (uint32_t)kq <= (uint32_t)kKMax) {
      // K holds exactly k entries: gather their keys and masses, then each
      // member's mass above it (strictly larger keys: whole tie groups) decides
      // P directly -- j in P iff mass(K, key > key_j) < p * mass(K).  The
      // smallest key in P is the cutoff; the sums are the same integers as
      // the radix select's, so the cutoff is too.
      if (tid == 0) {
        sh.nk = 0;
        sh.vcmin = 0xFFFFFFFFu;
      }
      __syncthreads();
      for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t k = Key::from_bits(raw[i]);
          if (in_k(k, j0 + i)) {
            const uint32_t slot = atomicAdd(&sh.nk, 1u);
            if (slot < (uint32_t)kKMax) {
              sh.kkey[slot] = k;
              sh.kmass[slot] = fixed_mass(raw[i]);
            }
          }
        }
      });
      __syncthreads();
      const uint32_t nk = sh.nk < (uint32_t)kKMax ? sh.nk : (uint32_t)kKMax;
      const unsigned long long zk = block_sum_u64((uint32_t)tid < nk ? sh.kmass[tid] : 0ull, sh);
      const double target = (double)pq * (double)zk;
      if ((uint32_t)tid < nk) {
        // four members per 16-byte key read, several reads in flight (one
        // shared-memory read per iteration would wait out its latency each time)
        const uint4* k4 = reinterpret_cast<const uint4*>(sh.kkey);
        const ulonglong2* m2 = reinterpret_cast<const ulonglong2*>(sh.kmass);
        const uint32_t kt = sh.kkey[tid];
        unsigned long long above = 0;
#pragma unroll 4
        for (uint32_t i = 0; i < nk; i += 4) {
          const uint4 kk = k4[i >> 2];
          const ulonglong2 ma = m2[i >> 1];
          const ulonglong2 mb = m2[(i >> 1) + 1];
          above += (kk.x > kt ? ma.x : 0ull) + (i + 1 < nk && kk.y > kt ? ma.y : 0ull) +
                   (i + 2 < nk && kk.z > kt ? mb.x : 0ull) + (i + 3 < nk && kk.w > kt ? mb.y : 0ull);
        }
        if ((double)above < target) atomicMin(&sh.vcmin, kt);
      }
      __syncthreads();
      vc = sh.vcmin;
    } else {
      uint32_t prefix = 0, pmask = 0;
      unsigned long long above = 0, bin = 0;
      double target = 0.0;
      for (int shift = Key::kBits - 8; shift >= 0; shift -= 8) {
        if (tid < 256) sh.hist64[tid] = 0;
        __syncthreads();
        for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k = Key::from_bits(raw[i]);
            if (in_k(k, j0 + i) && (k & pmask) == prefix)
              atomicAdd(&sh.hist64[(k >> shift) & 255u], fixed_mass(raw[i]));
          }
        });
        __syncthreads();
        if (shift == Key::kBits - 8) {
          const int lane = tid & (kWave - 1);
          unsigned long long z = sh.hist64[4 * lane] + sh.hist64[4 * lane + 1] +
                                 sh.hist64[4 * lane + 2] + sh.hist64[4 * lane + 3];
          z = wave_sum(z);
          target = (double)pq * (double)z;
        }
        const int d = find_digit_desc<unsigned long long>(
            sh.hist64, above, [&](unsigned long long c) { return (double)c >= target; }, &above,
            &bin);
        prefix |= (uint32_t)d << shift;
        pmask |= 255u << shift;
        __syncthreads();
      }
      vc = prefix;
    }
  }
  auto in_p = [&](uint32_t k, int64_t j) -> bool { return in_k(k, j) && (!p_on || k >= vc); };

  // ---- F: mass of P, then noise + argmax (sample) or the log-prob write.
  if (MODE == kOutSample) {
    const uint64_t off = noise_offset(a, q);
    const NoiseStream ns{(uint32_t)a.seed[q], (uint32_t)(a.seed[q] >> 32), (uint32_t)r,
                         (uint32_t)off, (uint32_t)(off >> 32)};
    ArgBest best{-__builtin_inff(), 0x7FFFFFFF};
    unsigned long long zp = 0;
    for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
      bool any = false;
      bool mem[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mem[i] = in_p(Key::from_bits(raw[i]), j0 + i);
        any |= mem[i];
      }
      if (!any) return;
      const Philox4 b = ns.block((uint32_t)(j0 >> 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!mem[i]) continue;
        zp += fixed_mass(raw[i]);
        const float z = __fmul_rn(E::value(raw[i]), inv_t) + gumbel_from_word(b.v[i]);
        if (better(z, (int32_t)(j0 + i), best.z, best.j)) best = ArgBest{z, (int32_t)(j0 + i)};
      }
    });
    zp = block_sum_u64(zp, sh);
    best = block_argbest(best, sh);
    if (tid == 0) {
      if (best.j < 0 || (int64_t)best.j >= v) {   // unreachable: P always holds the top entry
        a.out_ids[r] = -1;
        if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
        return;
      }
      a.out_ids[r] = best.j;
      if (a.out_lp) {
        uint32_t raw[4];
        E::load4(row, best.j, best.j + 1, false, raw);
        const float s = __fmul_rn(E::value(raw[0]), inv_t);
        const double lz = log((double)zp) - (double)a.mass_shift * 0.69314718055994530942;
        a.out_lp[r] = (float)((double)s - (double)m - lz);
      }
    }
    return;
  }

  unsigned long long zp = 0;
  for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (in_p(Key::from_bits(raw[i]), j0 + i)) zp += fixed_mass(raw[i]);
  });
  zp = block_sum_u64(zp, sh);
  const float lz = (float)(log((double)zp) - (double)a.mass_shift * 0.69314718055994530942);
  if (MODE == kOutLogProbAt) {
    if (tid == 0) {
      const int64_t j = a.token_ids[r];
      float out = -__builtin_inff();
      if (j >= 0 && j < v) {
        uint32_t raw[4];
        E::load4(row, j, j + 1, false, raw);
        if (in_p(Key::from_bits(raw[0]), j)) out = __fmul_rn(E::value(raw[0]), inv_t) - m - lz;
      }
      a.out_lp[r] = out;
    }
    return;
  }
  float* out_row = a.out_lp + (int64_t)r * v;
  for_groups(row, v, vec, [&](int64_t j0, const uint32_t* raw) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (j0 + i >= v) break;
      const bool keep = in_p(Key::from_bits(raw[i]), j0 + i);
      out_row[j0 + i] = keep ? (__fmul_rn(E::value(raw[i]), inv_t) - m - lz) : -__builtin_inff();
    }
  });
}

}  // namespace general

}  // namespace tss
