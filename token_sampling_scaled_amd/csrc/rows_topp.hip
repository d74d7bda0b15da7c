// Top-p route (every row of the call filtered by top-p only, or unfiltered):
// two kernels.
//
// 1. rows_topp_cutoff_kernel, one workgroup of 1024 threads per row, three
//    passes over the row (the first from HBM, the others mostly from the
//    Infinity Cache):
//    a. max m and Z = sum exp2(s - m) of s = x log2(e) / T (online, per
//       thread), and the first maximum for greedy rows;
//    b. a histogram of counts and fixed-point masses exp2(s - m) over 4096
//       equal buckets of s in [lo, m], where lo = m + log2((1 - p) Z / V): the
//       entries below lo weigh less than (1 - p) Z all together, so the top-p
//       cutoff is never below lo.  The first bucket (from the top) whose
//       cumulative mass reaches p Z holds the cutoff;
//    c. the order keys of that bucket's entries are gathered in LDS and a
//       radix select over them (11, 11 and 10 bits) on the cumulative mass
//       gives the exact cutoff key: the first tie group whose cumulative mass
//       reaches p Z.  If the bucket holds more entries than LDS does, the same
//       radix passes read them from the row instead.
//    The row's cutoff key and the mass of P go to the workspace.
// 2. rows_topp_draw_kernel, a grid of 256-thread workgroups taking (row, tile)
//    items in a fixed interleaved order: the 4-entry groups of a tile that
//    hold members of P (key >= cutoff key) are compacted in LDS, one Philox
//    block per group gives its members' noise, and the tile's perturbed argmax
//    is kept; the item that finishes a row last merges the row's tiles and
//    writes id and log-prob.
//
// Masses are 64-bit fixed-point integers (scale 2^mass_shift, plus one per
// entry so that a nonzero sum marks a nonempty bin), so every sum is
// independent of the order of the atomics.  Greedy rows and rows with no entry
// above -inf are finished by the first kernel.
#include "split_common.hpp"

namespace tss {

namespace {

using namespace split;

constexpr int kCutBlock = 1024;
constexpr int kCutWaves = kCutBlock / kWave;
constexpr int kBuckets = 4096;
constexpr int kCand = 16384;          // cutoff-bucket keys held in LDS
constexpr int kRadixBins = 2048;
constexpr uint32_t kModeCut = 0;      // draw from the entries with key >= key_c
constexpr uint32_t kModeDone = 1;     // result already written
constexpr int kDrawPT = 4;            // 4-entry groups per thread in a draw tile
constexpr int kDrawTile = kDrawPT * kSplitBlock;
constexpr int kDrawBlocks = 2048;     // persistent draw workgroups

template <typename T>
struct KeyRaw;
template <>
struct KeyRaw<float> {
  __device__ __forceinline__ static float value_of_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  }
};
template <>
struct KeyRaw<uint16_t> {
  __device__ __forceinline__ static float value_of_key(uint32_t k) {
    const uint32_t raw = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    return __uint_as_float(raw << 16);
  }
};

// Calls f(g, raw[4]) for every 4-entry group of the row this thread owns
// (groups tid, tid + 1024, ...), with eight groups' loads in flight at once.
template <typename T, bool VEC, typename F>
__device__ __forceinline__ void for_row_groups(const T* row, int64_t v, int32_t groups, F&& f) {
  using E = SplitElem<T>;
  constexpr int U = 8;
  for (int32_t g0 = (int32_t)threadIdx.x; g0 < groups; g0 += U * kCutBlock) {
    uint32_t raw[U][4];
    if (VEC) {
      typename E::Packed pk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t g = g0 + u * kCutBlock;
        pk[u] = *reinterpret_cast<const typename E::Packed*>(row + (int64_t)(g < groups ? g : groups - 1) * 4);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) E::unpack(pk[u], raw[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t g = g0 + u * kCutBlock;
        if (g < groups) {
          E::load4(row, (int64_t)g * 4, v, raw[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t g = g0 + u * kCutBlock;
      if (g < groups) f(g, raw[u]);
    }
  }
}

struct CutShared {
  unsigned long long mass[kBuckets];   // fixed-point masses, each entry + 1: 0 = empty
  uint32_t cand[kCand];
  unsigned long long wtot[kCutWaves];
  Lse wlse[kCutWaves];
  uint32_t wkey[kCutWaves];
  int32_t wj[kCutWaves];
  uint32_t ncand;
  int32_t hit;                    // crossing bin
  int32_t first;                  // first nonempty bin
  int32_t last;                   // last nonempty bin
  unsigned long long hit_above;   // mass of the bins above the crossing bin
  unsigned long long hit_mass;    // mass of the crossing bin
};

// In bins [0, nb) ordered from the largest values down, the first nonempty bin
// whose cumulative mass, on top of `base`, reaches `target` (the first
// nonempty bin when base already does); if none does, the last nonempty bin.  Writes the bin, the mass above it and its own mass to LDS
// (valid after the call, in every thread).
__device__ __forceinline__ void find_crossing(CutShared& sh, int nb, unsigned long long base,
                                              double target) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int per = nb / kCutBlock;            // 4 or 2 bins per thread
  unsigned long long mine = 0;
  int lastne = -1, firstne = 0x7FFFFFFF;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    mine += sh.mass[b];
    if (sh.mass[b]) {
      lastne = b;
      firstne = min(firstne, b);
    }
  }
  if (tid == 0) {
    sh.hit = -1;
    sh.last = -1;
    sh.first = 0x7FFFFFFF;
  }
  // inclusive scan over the wave, then over the waves
  unsigned long long incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sh.wtot[wid] = incl;
  __syncthreads();
  if (lastne >= 0) {
    atomicMax(&sh.last, lastne);
    atomicMin(&sh.first, firstne);
  }
  unsigned long long before = base + incl - mine;
  for (int w = 0; w < wid; ++w) before += sh.wtot[w];
  unsigned long long cum = before;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    const unsigned long long m = sh.mass[b];
    if ((double)(cum + m) >= target && (double)cum < target && m) {
      sh.hit = b;
      sh.hit_above = cum - base;
      sh.hit_mass = m;
    }
    cum += m;
  }
  __syncthreads();
  if ((double)base >= target) {
    // the mass above already reaches the target: only the first group stays
    if (tid == 0) {
      const int b = sh.first < nb ? sh.first : 0;
      sh.hit = b;
      sh.hit_above = 0;
      sh.hit_mass = sh.mass[b];
    }
    __syncthreads();
  } else if (sh.hit < 0) {
    // the target was not reached (rounding): take every nonempty bin
    if (tid == 0) {
      const int b = sh.last;
      unsigned long long above = 0;
      for (int w = 0; w < kCutWaves; ++w) above += sh.wtot[w];
      sh.hit = b;
      sh.hit_mass = b >= 0 ? sh.mass[b] : 0ull;
      sh.hit_above = above - sh.hit_mass;
    }
    __syncthreads();
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kCutBlock) void rows_topp_cutoff_kernel(RowArgs a) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ CutShared sh;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
  const int64_t q = a.req_map ? (int64_t)a.req_map[r] : (int64_t)r;
  const T* row = reinterpret_cast<const T*>(a.logits) + src * a.row_stride;
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  const float temp = a.temperature[q];
  const float p = a.top_p ? a.top_p[q] : 1.0f;
  const bool greedy = !(temp >= 1e-5f);
  const float scale2 = greedy ? 1.0f : 1.4426950408889634f / temp;
  const float fx_scale = __builtin_ldexpf(1.0f, a.mass_shift);
  TopPRow* st = a.topp_rows + r;

  // ---- a. max, log-sum-exp (base 2), first maximum for greedy rows
  float m = -__builtin_inff(), z = 0.0f;
  uint32_t bkey = 0;
  int32_t bj = 0x7FFFFFFF;
  for_row_groups<T, VEC>(row, v, groups, [&](int32_t g, const uint32_t (&raw)[4]) {
    if (greedy) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = K::from_bits(raw[e]);
        if (key > K::kNegInf && key > bkey) {   // groups rise within a thread
          bkey = key;
          bj = g * 4 + e;
        }
      }
      return;
    }
    float s[4];
    float gmx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = E::value(raw[e]);
      s[e] = x == x ? x * scale2 : -__builtin_inff();
      gmx = fmaxf(gmx, s[e]);
    }
    if (gmx > m) {
      z = (m == -__builtin_inff()) ? 0.0f : z * __builtin_amdgcn_exp2f(m - gmx);
      m = gmx;
    }
    if (m > -__builtin_inff()) {
#pragma unroll
      for (int e = 0; e < 4; ++e) z += __builtin_amdgcn_exp2f(s[e] - m);
    }
  });
  if (greedy) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t ok = (uint32_t)__shfl_xor((int)bkey, off, kWave);
      const int32_t oj = __shfl_xor(bj, off, kWave);
      if (ok > bkey || (ok == bkey && oj < bj)) {
        bkey = ok;
        bj = oj;
      }
    }
    if (lane == 0) {
      sh.wkey[wid] = bkey;
      sh.wj[wid] = bj;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kCutWaves; ++w) {
        if (sh.wkey[w] > bkey || (sh.wkey[w] == bkey && sh.wj[w] < bj)) {
          bkey = sh.wkey[w];
          bj = sh.wj[w];
        }
      }
      const bool none = bj == 0x7FFFFFFF;
      a.out_ids[r] = none ? -1 : bj;
      if (a.out_lp) a.out_lp[r] = none ? __builtin_nanf("") : 0.0f;
      st->mode = kModeDone;
    }
    return;
  }
  Lse l = wave_lse(Lse{m, z});
  if (lane == 0) sh.wlse[wid] = l;
  __syncthreads();
  l = sh.wlse[0];
  for (int w = 1; w < kCutWaves; ++w) l = lse_merge(l, sh.wlse[w]);
  const float m2 = l.m, z2 = l.sum;
  if (m2 == -__builtin_inff()) {             // no entry above -inf
    if (tid == 0) {
      a.out_ids[r] = -1;
      if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
      st->mode = kModeDone;
    }
    return;
  }
  if (!(p < 1.0f - 1e-6f)) {                 // filter off: P = every entry above -inf
    if (tid == 0) {
      st->mode = kModeCut;
      st->key_c = K::kNegInf + 1;
      st->m2 = m2;
      st->zp = z2;
      st->src = src;
      st->seed = a.seed[q];
      st->scale2 = scale2;
      st->off = noise_offset(a, q);
    }
    return;
  }

  // ---- b. histogram of the entries >= lo over 4096 buckets of s
  const float span = -__builtin_amdgcn_logf(fmaxf(1.0f - p, 0.0f) * z2 / (float)v);
  const float lo2 = (span > 0.0f) ? m2 - span : m2 - 1.0f;
  const float inv_w = (float)kBuckets / (m2 - lo2);
  for (int b = tid; b < kBuckets; b += kCutBlock) sh.mass[b] = 0;
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  auto bucket_of = [&](float s) -> int {
    const float f = (m2 - s) * inv_w;        // >= 0; NaN only if inv_w overflowed
    return f >= 0.0f ? (f < (float)(kBuckets - 1) ? (int)f : kBuckets - 1) : 0;
  };
  // an entry's fixed-point mass, plus one so that every counted entry shows
  // (the bias is at most V units against a scale of 2^mass_shift)
  auto fixed_mass = [&](float s) -> unsigned long long {
    return (unsigned long long)(__builtin_amdgcn_exp2f(s - m2) * fx_scale) + 1ull;
  };
  for_row_groups<T, VEC>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = E::value(raw[e]);
      const float s = x * scale2;
      if (x == x && s >= lo2) {
        atomicAdd(&sh.mass[bucket_of(s)], fixed_mass(s));
      }
    }
  });
  __syncthreads();
  const double target = (double)p * (double)z2 * (double)fx_scale;
  find_crossing(sh, kBuckets, 0ull, target);
  const int bstar = sh.hit;
  unsigned long long above = sh.hit_above;

  // ---- c. the cutoff bucket's keys, then a radix select on them
  for_row_groups<T, VEC>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = E::value(raw[e]);
      const float s = x * scale2;
      if (x == x && s >= lo2 && bucket_of(s) == bstar) {
        const uint32_t slot = atomicAdd(&sh.ncand, 1u);
        if (slot < (uint32_t)kCand) sh.cand[slot] = K::from_bits(raw[e]);
      }
    }
  });
  __syncthreads();
  const uint32_t nc = sh.ncand;
  const bool from_lds = nc <= (uint32_t)kCand;
  uint32_t prefix = 0;
  unsigned long long zp_fx = 0;
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBits[3] = {11, 11, 10};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass], bits = kBits[pass];
    const int nb = kRadixBins;
    for (int b = tid; b < nb; b += kCutBlock) sh.mass[b] = 0;
    __syncthreads();
    auto add_key = [&](uint32_t key) {
      if (pass > 0 && (key >> (shift + bits)) != prefix) return;
      const int d = (int)((key >> shift) & ((1u << bits) - 1u));
      const int b = (nb - 1) - d;          // bins from the largest digit down
      const float s = KeyRaw<T>::value_of_key(key) * scale2;
      atomicAdd(&sh.mass[b], fixed_mass(s));
    };
    if (from_lds) {
      for (uint32_t t = tid; t < nc; t += kCutBlock) add_key(sh.cand[t]);
    } else {
      for_row_groups<T, VEC>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = E::value(raw[e]);
          const float s = x * scale2;
          if (x == x && s >= lo2 && bucket_of(s) == bstar) add_key(K::from_bits(raw[e]));
        }
      });
    }
    __syncthreads();
    find_crossing(sh, nb, above, target);
    const int d = (nb - 1) - (sh.hit < 0 ? 0 : sh.hit);
    above += sh.hit_above;
    prefix = (prefix << bits) | (uint32_t)d;
    zp_fx = above + sh.hit_mass;
    __syncthreads();
  }
  if (tid == 0) {
    st->mode = kModeCut;
    st->key_c = prefix;
    st->m2 = m2;
    st->zp = (float)((double)zp_fx / (double)fx_scale);
    st->src = src;
    st->seed = a.seed[q];
    st->scale2 = scale2;
    st->off = noise_offset(a, q);
  }
}

// Draw: the (row, tile) items run tile by tile over all rows (every row's tile
// 0, then every row's tile 1, ...) and workgroup b takes items b, b + B, ...,
// so rows with a large P spread over many workgroups.  A tile is PT 4-entry
// groups per thread.  Each item leaves the best of its members as a partial;
// the item that takes a row's last ticket merges the row's partials in tile
// order and writes the id and the log-prob.
template <typename T, bool VEC, int PT>
__global__ __launch_bounds__(kSplitBlock) void rows_topp_draw_kernel(RowArgs a, int32_t ntiles) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  constexpr int kTile = PT * kSplitBlock;    // groups per tile
  __shared__ uint32_t mg[kTile];       // member groups: (group << 4) | member mask
  __shared__ float ms[kTile][4];       // their scaled logits
  __shared__ uint32_t woff[kSplitWaves + 1];
  __shared__ Best sbest[kSplitWaves];
  __shared__ uint32_t sticket;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  const uint32_t total = (uint32_t)a.n * (uint32_t)ntiles;

  for (uint32_t item = blockIdx.x; item < total; item += gridDim.x) {
    const int r = (int)(item % (uint32_t)a.n);
    const int tile = (int)(item / (uint32_t)a.n);
    const TopPRow* st = a.topp_rows + r;
    if (st->mode != kModeCut) continue;      // uniform over the workgroup
    const uint32_t key_c = st->key_c;
    const T* row = reinterpret_cast<const T*>(a.logits) + st->src * a.row_stride;
    const float scale2 = st->scale2;
    const uint64_t seed = st->seed;
    const uint64_t off = st->off;
    const NoiseStream ns{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r,
                         (uint32_t)off, (uint32_t)(off >> 32)};
    const int32_t t0 = tile * kTile;
    const int32_t t_end = t0 + kTile < groups ? t0 + kTile : groups;

    uint32_t raw[PT][4];
    if (VEC) {
      typename E::Packed pk[PT];
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int32_t g = t0 + tid + i * kSplitBlock;
        pk[i] = *reinterpret_cast<const typename E::Packed*>(row + (int64_t)(g < t_end ? g : t_end - 1) * 4);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < PT; ++i) E::unpack(pk[i], raw[i]);
    } else {
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int32_t g = t0 + tid + i * kSplitBlock;
        if (g < t_end) {
          E::load4(row, (int64_t)g * 4, v, raw[i]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) raw[i][e] = E::kNegInfRaw;
        }
      }
    }
    // 4-entry groups of this tile that hold members of P (key >= key_c),
    // compacted in LDS: one Philox block per such group gives the noise of all
    // its members
    uint32_t gmask[PT];
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const bool in = t0 + tid + i * kSplitBlock < t_end;
      gmask[i] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        gmask[i] |= (in && K::from_bits(raw[i][e]) >= key_c ? 1u : 0u) << e;
      cnt += gmask[i] ? 1u : 0u;
    }
    const uint32_t incl = wave_scan_incl(cnt);
    if (lane == kWave - 1) woff[wid + 1] = incl;
    __syncthreads();
    if (tid == 0) {
      woff[0] = 0;
      for (int w = 1; w <= kSplitWaves; ++w) woff[w] += woff[w - 1];
    }
    __syncthreads();
    uint32_t pos = woff[wid] + incl - cnt;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      if (gmask[i]) {
        mg[pos] = ((uint32_t)(t0 + tid + i * kSplitBlock) << 4) | gmask[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) ms[pos][e] = E::value(raw[i][e]) * scale2;
        ++pos;
      }
    }
    __syncthreads();
    const uint32_t nm = woff[kSplitWaves];
    float bz = -__builtin_inff();
    int32_t bj = 0x7FFFFFFF;
    float bs = 0.0f;
    for (uint32_t t = tid; t < nm; t += kSplitBlock) {
      const uint32_t gm = mg[t];
      const uint32_t g = gm >> 4;
      const Philox4 w = ns.block(g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!((gm >> e) & 1u)) continue;
        const float sv = ms[t][e];
        const float zz = sv + gumbel2_from_word(w.v[e]);
        const int32_t jj = (int32_t)(g * 4 + e);
        if (better(zz, jj, bz, bj)) {
          bz = zz;
          bj = jj;
          bs = sv;
        }
      }
    }
    Best best{0u, 0x7FFFFFFF, 0.0f};
    if (bz > -__builtin_inff()) best = Best{order_of(bz), bj, bs};
    best = wave_best(best);
    if (lane == 0) sbest[wid] = best;
    __syncthreads();
    SplitPartial* parts = reinterpret_cast<SplitPartial*>(a.split_partials) + (int64_t)r * ntiles;
    if (tid == 0) {
      Best b = sbest[0];
#pragma unroll
      for (int w = 1; w < kSplitWaves; ++w)
        if (beats(sbest[w].o, sbest[w].j, b.o, b.j)) b = sbest[w];
      SplitPartial* pp = parts + tile;
      store_agent(&pp->o, b.o);
      store_agent(&pp->j, b.j);
      store_agent(&pp->s, b.s);
      // see rows_split.hip: device-coherent stores, acknowledged, then the ticket
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      sticket = __hip_atomic_fetch_add(a.split_counter + r, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (sticket == (uint32_t)(ntiles - 1) && wid == 0) {
      Best b{0u, 0x7FFFFFFF, 0.0f};
      for (int p0 = 0; p0 < ntiles; p0 += kWave) {
        Best bb{0u, 0x7FFFFFFF, 0.0f};
        if (p0 + lane < ntiles) {
          const SplitPartial* pp = parts + p0 + lane;
          bb = Best{load_agent_u(&pp->o), load_agent_i(&pp->j), load_agent_f(&pp->s)};
        }
        bb = wave_best(bb);
        if (beats(bb.o, bb.j, b.o, b.j)) b = bb;
      }
      if (lane == 0) {
        if (b.j == 0x7FFFFFFF) {      // cannot happen: P holds the row maximum
          a.out_ids[r] = -1;
          if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
        } else {
          a.out_ids[r] = b.j;
          if (a.out_lp)
            a.out_lp[r] = (b.s - st->m2 - __builtin_amdgcn_logf(st->zp)) * 0.69314718055994531f;
        }
        __hip_atomic_store(a.split_counter + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();                           // LDS lists and sticket are reused
  }
}

template <typename T, bool VEC>
hipError_t launch_typed(const RowArgs& a, int32_t ntiles, hipStream_t stream) {
  hipLaunchKernelGGL((rows_topp_cutoff_kernel<T, VEC>), dim3(a.n), dim3(kCutBlock), 0, stream, a);
  const int64_t items = (int64_t)a.n * ntiles;
  const uint32_t blocks = (uint32_t)(items < kDrawBlocks ? items : kDrawBlocks);
  hipLaunchKernelGGL((rows_topp_draw_kernel<T, VEC, kDrawPT>), dim3(blocks), dim3(kSplitBlock), 0,
                     stream, a, ntiles);
  return hipGetLastError();
}

}  // namespace

bool topp_supported(const RowArgs& a) {
  const int64_t groups = (a.vocab + 3) >> 2;
  const int64_t tiles = (groups + kDrawTile - 1) / kDrawTile;
  return a.topp_rows != nullptr && a.split_counter != nullptr &&
         a.split_partials != nullptr && tiles <= kMaxSplit;
}

hipError_t launch_rows_topp(const RowArgs& a, DType dtype, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int64_t groups = (a.vocab + 3) >> 2;
  const int32_t ntiles = (int32_t)((groups + kDrawTile - 1) / kDrawTile);
  const uintptr_t base = reinterpret_cast<uintptr_t>(a.logits);
  if (dtype == kF32) {
    const bool vec = (base % 16) == 0 && (a.row_stride % 4) == 0 && (a.vocab % 4) == 0;
    return vec ? launch_typed<float, true>(a, ntiles, stream)
               : launch_typed<float, false>(a, ntiles, stream);
  }
  const bool vec = (base % 8) == 0 && (a.row_stride % 4) == 0 && (a.vocab % 4) == 0;
  return vec ? launch_typed<uint16_t, true>(a, ntiles, stream)
             : launch_typed<uint16_t, false>(a, ntiles, stream);
}

}  // namespace tss
