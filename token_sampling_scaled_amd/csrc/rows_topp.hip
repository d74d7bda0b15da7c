// Top-p route (every row of the call filtered by top-p only, or unfiltered):
// three kernels; the row is read once from HBM and once more by the draw
// (mostly from the Infinity Cache, which still holds it).
//
// 1. rows_topp_hist_kernel, one workgroup of 1024 threads per row:
//    - mass reference m0 = the largest scaled logit s2 = x log2(e) / T among
//      the first eight 4-entry groups of every thread (read before anything
//      else);
//    - Z = the row's mass: every entry above -inf weighs
//      floor(exp2(s2 - m0) 2^shift) + 1 (64-bit fixed point, so every sum is
//      independent of the order of the additions);
//    - with top-p on, a histogram of those masses over kBuckets equal buckets
//      of s2 in [top2 - span, top2], counted from the top: top2 = m0 + 8,
//      span = 9 + max(0, log2(V / (1 - p))).  The entries below that range weigh less
//      than (1 - p) Z all together (Z is at least the mass of the row's
//      maximum, which lies within 8 of m0), so the top-p cutoff lies inside
//      it.  The first nonempty bucket from the top whose cumulative mass
//      reaches p Z holds the cutoff tie group: bucket b*.  A row whose maximum
//      exceeds top2 repeats the pass with m0 = its maximum.
// 2. rows_topp_draw_kernel, (row, tile) workgroups of 256 threads: the
//    entries in buckets above b* are members of P; each 4-entry group holding
//    a member, or an entry of b*, draws one Philox block.  Entries of b* are
//    appended (order key, index, perturbed score) to the row's list.  Each tile
//    leaves its best member as a partial result.
// 3. rows_topp_finish_kernel, one workgroup per row: the exact cutoff inside
//    b* from the list -- the largest key v whose entries at or above v, with
//    the mass above b*, reach p Z (so whole tie groups stay together) -- then
//    the best of the tiles and of the list's members, the id and its log-prob.
//    A list that overflowed its capacity is rebuilt from the row by radix
//    passes over the order keys of b*.
// Greedy rows and rows with no entry above -inf are finished by the first
// kernel.
#include "split_common.hpp"

namespace tss {

namespace {

using namespace split;

constexpr int kHistBlock = 1024;
constexpr int kHistWaves = kHistBlock / kWave;
constexpr int kBuckets = 16384;
constexpr int kBucketsPerThread = kBuckets / kHistBlock;
constexpr float kHeadroom = 8.0f;     // base-2 units of s2 above m0 covered by the histogram
constexpr int kFirstBatch = 8;        // groups per thread read before m0 is fixed
constexpr int kDrawPT = 8;            // 4-entry groups per thread in a draw tile
constexpr int kDrawTile = kDrawPT * kSplitBlock;
constexpr int kCand = 16384;          // cutoff-bucket keys held in LDS (overflow path)
constexpr int kRadixBins = 2048;

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

// Scaled logit s2 = x log2(e) / T, -inf for NaN.  Rounded products and
// differences only (no contraction), so every kernel that recomputes a bucket
// or a mass from the same entry gets the same bits.
__device__ __forceinline__ float scaled2(float x, float scale2) {
  return x == x ? __fmul_rn(x, scale2) : -__builtin_inff();
}

// Bucket of a scaled logit: 0 .. kBuckets - 1 inside the histogram's range,
// kBuckets below it (or -inf), -1 above its top.
__device__ __forceinline__ int bucket_of(float s2, float top2, float inv_w) {
  if (s2 > top2) return -1;
  const float f = __fmul_rn(__fsub_rn(top2, s2), inv_w);
  return f < (float)kBuckets ? (int)f : kBuckets;
}

// Fixed-point mass of an entry at most 2^8 above the reference (plus one, so
// that every counted entry shows in a sum).
__device__ __forceinline__ unsigned long long fixed_mass(float s2, float m0, float fx_scale) {
  return (unsigned long long)(__builtin_amdgcn_exp2f(__fsub_rn(s2, m0)) * fx_scale) + 1ull;
}

// 4-entry group g of the row (entries past the row read as -inf).
template <typename T, bool VEC>
__device__ __forceinline__ void load_group(const T* row, int64_t v, int32_t groups, int32_t g,
                                           uint32_t raw[4]) {
  using E = SplitElem<T>;
  if (VEC) {
    const typename E::Packed pk =
        *reinterpret_cast<const typename E::Packed*>(row + (int64_t)(g < groups ? g : groups - 1) * 4);
    E::unpack(pk, raw);
  } else if (g < groups) {
    E::load4(row, (int64_t)g * 4, v, raw);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[e] = E::kNegInfRaw;
  }
}

// Calls f(g, raw[4]) for every 4-entry group of the row this thread owns
// (groups tid, tid + B, ...), with eight groups' loads in flight at once.
template <typename T, bool VEC, int B, typename F>
__device__ __forceinline__ void for_row_groups(const T* row, int64_t v, int32_t groups, F&& f) {
  constexpr int U = 8;
  for (int32_t g0 = (int32_t)threadIdx.x; g0 < groups; g0 += U * B) {
    uint32_t raw[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) load_group<T, VEC>(row, v, groups, g0 + u * B, raw[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t g = g0 + u * B;
      if (g < groups) f(g, raw[u]);
    }
  }
}

__device__ __forceinline__ uint32_t lane_rank_u64(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// 1. histogram

struct HistShared {
  unsigned long long hist[kBuckets];
  unsigned long long wsum[kHistWaves];
  unsigned long long wscan[kHistWaves];
  float wmax[kHistWaves];
  uint32_t wovf[kHistWaves];
  uint32_t wkey[kHistWaves];
  int32_t wj[kHistWaves];
  int32_t hit;
  int32_t first;
  int32_t last;
  unsigned long long hit_above;
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kHistBlock) void rows_topp_hist_kernel(RowArgs a) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ HistShared sh;
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
  TopPRow* st = a.topp_rows + r;

  auto first_max = [&](bool nan_lp) {
    // first index of the largest order key (NaN as -inf, -0 as +0); greedy
    // rows, and rows whose maximum is +inf
    uint32_t bkey = 0;
    int32_t bj = 0x7FFFFFFF;
    for_row_groups<T, VEC, kHistBlock>(row, v, groups, [&](int32_t g, const uint32_t (&raw)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = K::from_bits(raw[e]);
        if (key > K::kNegInf && key > bkey) {   // groups rise within a thread
          bkey = key;
          bj = g * 4 + e;
        }
      }
    });
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
      for (int w = 1; w < kHistWaves; ++w) {
        if (sh.wkey[w] > bkey || (sh.wkey[w] == bkey && sh.wj[w] < bj)) {
          bkey = sh.wkey[w];
          bj = sh.wj[w];
        }
      }
      const bool none = bj == 0x7FFFFFFF;
      a.out_ids[r] = none ? -1 : bj;
      if (a.out_lp) a.out_lp[r] = (none || nan_lp) ? __builtin_nanf("") : 0.0f;
      st->mode = kTopPDone;
    }
  };
  if (greedy) {
    first_max(false);
    return;
  }

  const float scale2 = 1.4426950408889634f / temp;
  const bool p_on = p < 1.0f - 1e-6f;
  const int shift = 53 - a.index_bits < 40 ? 53 - a.index_bits : 40;
  const float fx_scale = __builtin_ldexpf(1.0f, shift);
  // histogram range below top2, in base-2 units: always at least the headroom
  // and one more, so the row maximum lies inside it
  const float span = kHeadroom + 1.0f +
                     fmaxf(__builtin_amdgcn_logf((float)v / fmaxf(1.0f - p, 1e-30f)), 0.0f);
  const float inv_w = (float)kBuckets / span;

  // ---- mass reference: the largest s2 among the first groups of every thread
  uint32_t first[kFirstBatch][4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < kFirstBatch; ++u) {
    const int32_t g = tid + u * kHistBlock;
    load_group<T, VEC>(row, v, groups, g, first[u]);
  }
  if (p_on) {
    for (int b = tid; b < kBuckets; b += kHistBlock) sh.hist[b] = 0ull;
  }
#pragma unroll
  for (int u = 0; u < kFirstBatch; ++u) {
    if (tid + u * kHistBlock >= groups) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, scaled2(E::value(first[u][e]), scale2));
  }
  tmax = wave_max_f(tmax);
  if (lane == 0) sh.wmax[wid] = tmax;
  __syncthreads();
  float m0 = sh.wmax[0];
  for (int w = 1; w < kHistWaves; ++w) m0 = fmaxf(m0, sh.wmax[w]);

  // ---- the pass: Z, the histogram, the row maximum, and whether any entry
  // lies above top2
  unsigned long long zt = 0;
  bool ovf = false;
  auto add_entries = [&](const uint32_t (&raw)[4], float m0v, float top2v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s2 = scaled2(E::value(raw[e]), scale2);
      tmax = fmaxf(tmax, s2);
      if (!(s2 > -__builtin_inff())) continue;
      if (s2 > top2v) {
        ovf = true;
        continue;
      }
      const unsigned long long fx = fixed_mass(s2, m0v, fx_scale);
      zt += fx;
      if (p_on) {
        const int b = bucket_of(s2, top2v, inv_w);
        if (b < kBuckets) atomicAdd(&sh.hist[b], fx);
      }
    }
  };
  float top2 = m0 + kHeadroom;
  {
#pragma unroll
    for (int u = 0; u < kFirstBatch; ++u)
      if (tid + u * kHistBlock < groups) add_entries(first[u], m0, top2);
    const int32_t g_rest = tid + kFirstBatch * kHistBlock;
    constexpr int U = 8;
    for (int32_t g0 = g_rest; g0 < groups; g0 += U * kHistBlock) {
      uint32_t raw[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) load_group<T, VEC>(row, v, groups, g0 + u * kHistBlock, raw[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (g0 + u * kHistBlock < groups) add_entries(raw[u], m0, top2);
    }
  }
  auto reduce = [&]() {
    const unsigned long long zw = wave_sum_u64(zt);
    const float mw = wave_max_f(tmax);
    const uint32_t ow = __ballot(ovf) ? 1u : 0u;
    __syncthreads();   // the previous readers of the wave slots are done
    if (lane == 0) {
      sh.wsum[wid] = zw;
      sh.wmax[wid] = mw;
      sh.wovf[wid] = ow;
    }
    __syncthreads();
  };
  reduce();
  float mrow = -__builtin_inff();
  bool any_ovf = false;
  for (int w = 0; w < kHistWaves; ++w) {
    mrow = fmaxf(mrow, sh.wmax[w]);
    any_ovf = any_ovf || sh.wovf[w] != 0;
  }
  if (mrow == -__builtin_inff()) {            // no entry above -inf
    if (tid == 0) {
      a.out_ids[r] = -1;
      if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
      st->mode = kTopPDone;
    }
    return;
  }
  if (mrow == __builtin_inff()) {             // +inf in the row: the first one, lp NaN
    __syncthreads();
    first_max(true);
    return;
  }
  if (any_ovf) {
    // the maximum lies more than the headroom above m0: the pass again with
    // m0 = the row maximum (re-read from the caches)
    m0 = mrow;
    top2 = m0 + kHeadroom;
    zt = 0;
    ovf = false;
    if (p_on) {
      for (int b = tid; b < kBuckets; b += kHistBlock) sh.hist[b] = 0ull;
    }
    __syncthreads();
    for_row_groups<T, VEC, kHistBlock>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
      add_entries(raw, m0, top2);
    });
    reduce();
  }
  unsigned long long z = 0;
  for (int w = 0; w < kHistWaves; ++w) z += sh.wsum[w];

  const uint64_t off = noise_offset(a, q);
  if (!p_on) {                                // P = every entry above -inf
    if (tid == 0) {
      st->mode = kTopPAll;
      st->m0 = m0;
      st->scale2 = scale2;
      st->shift = shift;
      st->above = z;
      st->src = src;
      st->seed = a.seed[q];
      st->off = off;
    }
    return;
  }

  // ---- the cutoff bucket: the first nonempty bucket from the top whose
  // cumulative mass reaches p Z (the first nonempty one when p <= 0; the last
  // nonempty one if rounding leaves the target unreached)
  const double target = (double)p * (double)z;
  unsigned long long mine = 0;
  int firstne = 0x7FFFFFFF, lastne = -1;
#pragma unroll
  for (int i = 0; i < kBucketsPerThread; ++i) {
    const int b = tid * kBucketsPerThread + i;
    const unsigned long long h = sh.hist[b];
    mine += h;
    if (h) {
      firstne = min(firstne, b);
      lastne = b;
    }
  }
  unsigned long long incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) sh.wscan[wid] = incl;
  if (tid == 0) {
    sh.hit = -1;
    sh.first = 0x7FFFFFFF;
    sh.last = -1;
  }
  __syncthreads();
  if (lastne >= 0) {
    atomicMin(&sh.first, firstne);
    atomicMax(&sh.last, lastne);
  }
  unsigned long long cum = incl - mine;
  for (int w = 0; w < wid; ++w) cum += sh.wscan[w];
#pragma unroll
  for (int i = 0; i < kBucketsPerThread; ++i) {
    const int b = tid * kBucketsPerThread + i;
    const unsigned long long h = sh.hist[b];
    if (h && (double)cum < target && (double)(cum + h) >= target) {
      sh.hit = b;
      sh.hit_above = cum;
    }
    cum += h;
  }
  __syncthreads();
  if (tid == 0) {
    int bstar = sh.hit;
    unsigned long long above = sh.hit_above;
    if (bstar < 0) {
      if (target <= 0.0) {
        bstar = sh.first < kBuckets ? sh.first : 0;
        above = 0;
      } else {
        bstar = sh.last >= 0 ? sh.last : 0;
        unsigned long long tot = 0;
        for (int w = 0; w < kHistWaves; ++w) tot += sh.wscan[w];
        above = tot - sh.hist[bstar];
      }
    }
    st->mode = kTopPCut;
    st->bstar = bstar;
    st->top2 = top2;
    st->inv_w = inv_w;
    st->m0 = m0;
    st->scale2 = scale2;
    st->shift = shift;
    st->nlist = 0;
    st->above = above;
    st->target = target;
    st->src = src;
    st->seed = a.seed[q];
    st->off = off;
  }
}

// ---------------------------------------------------------------------------
// 2. draw

// Tile `tile` of row r: members of P (buckets above b*, or every entry above
// -inf when P is the whole row) and the entries of b*; each wave compacts its
// groups that hold one, then draws one Philox block per compacted group.
template <typename T, bool VEC, int PT>
__global__ __launch_bounds__(kSplitBlock) void rows_topp_draw_kernel(RowArgs a, int32_t ntiles) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ uint32_t cg[kSplitWaves][PT * kWave];        // group << 8 | boundary mask << 4 | member mask
  __shared__ uint32_t craw[kSplitWaves][PT * kWave][4];   // the group's raw entries
  __shared__ Best sbest[kSplitWaves];

  const int r = (int)(blockIdx.x % (uint32_t)a.n);
  const int tile = (int)(blockIdx.x / (uint32_t)a.n);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  TopPRow* st = a.topp_rows + r;
  const uint32_t mode = st->mode;
  if (mode == kTopPDone) return;                 // uniform over the workgroup
  const bool all = mode == kTopPAll;
  const int bstar = st->bstar;
  const float top2 = st->top2;
  const float inv_w = st->inv_w;
  const float scale2 = st->scale2;
  const T* row = reinterpret_cast<const T*>(a.logits) + st->src * a.row_stride;
  const uint64_t seed = st->seed;
  const uint64_t off = st->off;
  const NoiseStream ns{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r, (uint32_t)off,
                       (uint32_t)(off >> 32)};
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  const int32_t t0 = tile * kDrawTile;
  const int32_t t_end = t0 + kDrawTile < groups ? t0 + kDrawTile : groups;

  uint32_t raw[PT][4];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int32_t g = t0 + tid + i * kSplitBlock;
    load_group<T, VEC>(row, v, t_end, g, raw[i]);
  }
  uint32_t fill = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int32_t g = t0 + tid + i * kSplitBlock;
    uint32_t mm = 0, bm = 0;
    if (g < t_end) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s2 = scaled2(E::value(raw[i][e]), scale2);
        if (all) {
          mm |= (s2 > -__builtin_inff() ? 1u : 0u) << e;
        } else {
          const int b = bucket_of(s2, top2, inv_w);
          mm |= (b < bstar ? 1u : 0u) << e;
          bm |= (b == bstar ? 1u : 0u) << e;
        }
      }
    }
    const bool has = (mm | bm) != 0;
    const unsigned long long bal = __ballot(has);
    if (has) {
      const uint32_t pos = fill + lane_rank_u64(bal);
      cg[wid][pos] = ((uint32_t)g << 8) | (bm << 4) | mm;
#pragma unroll
      for (int e = 0; e < 4; ++e) craw[wid][pos][e] = raw[i][e];
    }
    fill += (uint32_t)__popcll(bal);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  Best best{0u, 0x7FFFFFFF, 0.0f};
  TopPCand* list = a.topp_list + (int64_t)r * kTopPListCap;
  for (uint32_t t = lane; t < fill; t += kWave) {
    const uint32_t c = cg[wid][t];
    const uint32_t g = c >> 8;
    const Philox4 w = ns.block(g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool mem = (c >> e) & 1u;
      const bool bnd = (c >> (4 + e)) & 1u;
      if (!(mem || bnd)) continue;
      const uint32_t rw = craw[wid][t][e];
      const float s2 = scaled2(E::value(rw), scale2);
      const float z2 = s2 + gumbel2_from_word(w.v[e]);
      const int32_t j = (int32_t)(g * 4 + e);
      if (mem) {
        const uint32_t o = order_of(z2);
        if (beats(o, j, best.o, best.j)) best = Best{o, j, s2};
      } else {
        const uint32_t slot = atomicAdd(&st->nlist, 1u);
        if (slot < (uint32_t)kTopPListCap) list[slot] = TopPCand{K::from_bits(rw), j, z2, s2};
      }
    }
  }
  best = wave_best(best);
  if (lane == 0) sbest[wid] = best;
  __syncthreads();
  if (tid == 0) {
    Best b = sbest[0];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w)
      if (beats(sbest[w].o, sbest[w].j, b.o, b.j)) b = sbest[w];
    SplitPartial* pp = reinterpret_cast<SplitPartial*>(a.split_partials) + (int64_t)r * ntiles + tile;
    pp->o = b.o;
    pp->j = b.j;
    pp->s = b.s;
  }
}

// ---------------------------------------------------------------------------
// 3. finish

struct FinShared {
  unsigned long long mass[kRadixBins];   // radix bins (overflow path)
  uint32_t cand[kCand];
  unsigned long long wtot[kHistWaves];
  Best wbest[kHistWaves];
  uint32_t ncand;
  int32_t hit;
  int32_t first;
  int32_t last;
  unsigned long long hit_above;
  unsigned long long hit_mass;
};

// In bins [0, nb) ordered from the largest keys down, the first nonempty bin
// whose cumulative mass, on top of `base`, reaches `target` (the first
// nonempty bin when base already does; the last nonempty bin if none does).
// Writes the bin, the mass above it and its own mass to LDS (valid after the
// call in every thread).
__device__ __forceinline__ void find_crossing(FinShared& sh, int nb, unsigned long long base,
                                              double target) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int per = nb / kHistBlock;
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
  unsigned long long incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) sh.wtot[wid] = incl;
  __syncthreads();
  if (lastne >= 0) {
    atomicMax(&sh.last, lastne);
    atomicMin(&sh.first, firstne);
  }
  unsigned long long cum = base + incl - mine;
  for (int w = 0; w < wid; ++w) cum += sh.wtot[w];
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    const unsigned long long m = sh.mass[b];
    if (m && (double)cum < target && (double)(cum + m) >= target) {
      sh.hit = b;
      sh.hit_above = cum - base;
      sh.hit_mass = m;
    }
    cum += m;
  }
  __syncthreads();
  if ((double)base >= target) {
    if (tid == 0) {
      const int b = sh.first < nb ? sh.first : 0;
      sh.hit = b;
      sh.hit_above = 0;
      sh.hit_mass = sh.mass[b];
    }
    __syncthreads();
  } else if (sh.hit < 0) {
    if (tid == 0) {
      const int b = sh.last;
      unsigned long long tot = 0;
      for (int w = 0; w < kHistWaves; ++w) tot += sh.wtot[w];
      sh.hit = b;
      sh.hit_mass = b >= 0 ? sh.mass[b] : 0ull;
      sh.hit_above = tot - sh.hit_mass;
    }
    __syncthreads();
  }
}

// id and log-prob: lp = (s2 - log2(sum over P of exp2(s2))) ln 2, with the sum
// held as zp = sum of fixed-point masses (scale 2^shift, reference m0).
__device__ __forceinline__ void write_row(const RowArgs& a, int r, const Best& b, float m0,
                                          unsigned long long zp, int shift) {
  if (b.j == 0x7FFFFFFF) {            // cannot happen: P holds the row maximum
    a.out_ids[r] = -1;
    if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
    return;
  }
  a.out_ids[r] = b.j;
  if (a.out_lp) {
    const float lz = __builtin_amdgcn_logf((float)zp) - (float)shift;
    a.out_lp[r] = (b.s - m0 - lz) * 0.69314718055994531f;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kHistBlock) void rows_topp_finish_kernel(RowArgs a, int32_t ntiles) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ FinShared sh;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const TopPRow* st = a.topp_rows + r;
  const uint32_t mode = st->mode;
  if (mode == kTopPDone) return;
  const float m0 = st->m0;
  const float scale2 = st->scale2;
  const float fx_scale = __builtin_ldexpf(1.0f, st->shift);
  const unsigned long long above = st->above;
  const uint32_t nlist = mode == kTopPCut ? st->nlist : 0u;
  const bool overflow = nlist > (uint32_t)kTopPListCap;

  // best of the tiles (wave 0)
  Best tb{0u, 0x7FFFFFFF, 0.0f};
  if (wid == 0) {
    const SplitPartial* parts = reinterpret_cast<const SplitPartial*>(a.split_partials) +
                                (int64_t)r * ntiles;
    for (int t0 = 0; t0 < ntiles; t0 += kWave) {
      Best b{0u, 0x7FFFFFFF, 0.0f};
      if (t0 + lane < ntiles) {
        const SplitPartial* pp = parts + t0 + lane;
        b = Best{pp->o, pp->j, pp->s};
      }
      b = wave_best(b);
      if (beats(b.o, b.j, tb.o, tb.j)) tb = b;
    }
  }
  if (mode == kTopPAll) {
    if (tid == 0) write_row(a, r, tb, m0, above, st->shift);
    return;
  }
  const double target = st->target;

  if (!overflow) {
    // ---- the list holds every entry of b*: one wave finds the cutoff key
    // v* = the largest key with (entries >= v* exist and) above + mass(>= v*)
    // >= target, by a bitwise descent from the leading bits all keys share
    if (wid != 0) return;
    constexpr int kPer = kTopPListCap / kWave;
    const TopPCand* list = a.topp_list + (int64_t)r * kTopPListCap;
    uint32_t key[kPer];
    unsigned long long fx[kPer];
    uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t t = (uint32_t)(i * kWave + lane);
      key[i] = 0;
      fx[i] = 0;
      if (t < nlist) {
        key[i] = list[t].key;
        fx[i] = fixed_mass(list[t].s2, m0, fx_scale);
        kmax = max(kmax, key[i]);
        kmin = min(kmin, key[i]);
      }
    }
    kmax = wave_max_u32(kmax);
    kmin = wave_min_u32(kmin);
    auto reach = [&](uint32_t trial) -> bool {
      unsigned long long m = 0;
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if ((uint32_t)(i * kWave + lane) < nlist && key[i] >= trial) {
          m += fx[i];
          ++c;
        }
      }
      m = wave_sum_u64(m);
      c = (uint32_t)__popcll(__ballot(c != 0));
      return c != 0 && (double)(above + m) >= target;
    };
    uint32_t vstar = kmin;              // kmin always reaches: every entry counts
    if (nlist > 0 && kmax != kmin) {
      const uint32_t diff = kmax ^ kmin;
      const int top = 31 - __builtin_clz(diff);
      uint32_t prefix = kmax & ~((2u << top) - 1u);
      for (int b = top; b >= 0; --b) {
        const uint32_t trial = prefix | (1u << b);
        if (reach(trial)) prefix = trial;
      }
      vstar = prefix < kmin ? kmin : prefix;
    } else if (nlist > 0) {
      vstar = kmax;
    }
    unsigned long long zp = 0;
    Best lb{0u, 0x7FFFFFFF, 0.0f};
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t t = (uint32_t)(i * kWave + lane);
      if (t < nlist && key[i] >= vstar) {
        zp += fx[i];
        const TopPCand c = list[t];
        const uint32_t o = order_of(c.z2);
        if (beats(o, c.j, lb.o, lb.j)) lb = Best{o, c.j, c.s2};
      }
    }
    zp = wave_sum_u64(zp);
    lb = wave_best(lb);
    if (beats(lb.o, lb.j, tb.o, tb.j)) tb = lb;
    if (lane == 0) write_row(a, r, tb, m0, above + zp, st->shift);
    return;
  }

  // ---- overflow: the order keys of b*'s entries from the row (gathered in
  // LDS when they fit), a radix select over them on the cumulative mass, then
  // the noise of b*'s members of P from the row
  const int bstar = st->bstar;
  const float top2 = st->top2;
  const float inv_w = st->inv_w;
  const T* row = reinterpret_cast<const T*>(a.logits) + st->src * a.row_stride;
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  for_row_groups<T, VEC, kHistBlock>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (bucket_of(scaled2(E::value(raw[e]), scale2), top2, inv_w) == bstar) {
        const uint32_t slot = atomicAdd(&sh.ncand, 1u);
        if (slot < (uint32_t)kCand) sh.cand[slot] = K::from_bits(raw[e]);
      }
    }
  });
  __syncthreads();
  const uint32_t nc = sh.ncand;
  const bool from_lds = nc <= (uint32_t)kCand;
  uint32_t prefix = 0;
  unsigned long long base = above, zp_fx = 0;
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBits[3] = {11, 11, 10};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shf = kShift[pass], bits = kBits[pass];
    for (int b = tid; b < kRadixBins; b += kHistBlock) sh.mass[b] = 0;
    __syncthreads();
    auto add_key = [&](uint32_t key) {
      if (pass > 0 && (key >> (shf + bits)) != prefix) return;
      const int d = (int)((key >> shf) & ((1u << bits) - 1u));
      const float s2 = __fmul_rn(KeyRaw<T>::value_of_key(key), scale2);
      atomicAdd(&sh.mass[(kRadixBins - 1) - d], fixed_mass(s2, m0, fx_scale));
    };
    if (from_lds) {
      for (uint32_t t = tid; t < nc; t += kHistBlock) add_key(sh.cand[t]);
    } else {
      for_row_groups<T, VEC, kHistBlock>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (bucket_of(scaled2(E::value(raw[e]), scale2), top2, inv_w) == bstar)
            add_key(K::from_bits(raw[e]));
      });
    }
    __syncthreads();
    find_crossing(sh, kRadixBins, base, target);
    const int d = (kRadixBins - 1) - (sh.hit < 0 ? 0 : sh.hit);
    base += sh.hit_above;
    prefix = (prefix << bits) | (uint32_t)d;
    zp_fx = base + sh.hit_mass;
    __syncthreads();
  }
  const uint32_t vstar = prefix;
  const NoiseStream ns{(uint32_t)st->seed, (uint32_t)(st->seed >> 32), (uint32_t)r,
                       (uint32_t)st->off, (uint32_t)(st->off >> 32)};
  Best b{0u, 0x7FFFFFFF, 0.0f};
  for_row_groups<T, VEC, kHistBlock>(row, v, groups, [&](int32_t g, const uint32_t (&raw)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s2 = scaled2(E::value(raw[e]), scale2);
      if (bucket_of(s2, top2, inv_w) != bstar || K::from_bits(raw[e]) < vstar) continue;
      const int32_t j = g * 4 + e;
      const float z2 = s2 + gumbel2_from_word(ns.word((uint32_t)j));
      const uint32_t o = order_of(z2);
      if (beats(o, j, b.o, b.j)) b = Best{o, j, s2};
    }
  });
  b = wave_best(b);
  if (lane == 0) sh.wbest[wid] = b;
  __syncthreads();
  if (tid == 0) {
    for (int w = 0; w < kHistWaves; ++w)
      if (beats(sh.wbest[w].o, sh.wbest[w].j, tb.o, tb.j)) tb = sh.wbest[w];
    write_row(a, r, tb, m0, zp_fx, st->shift);
  }
}

template <typename T, bool VEC>
hipError_t launch_typed(const RowArgs& a, int32_t ntiles, hipStream_t stream) {
  hipLaunchKernelGGL((rows_topp_hist_kernel<T, VEC>), dim3(a.n), dim3(kHistBlock), 0, stream, a);
  hipLaunchKernelGGL((rows_topp_draw_kernel<T, VEC, kDrawPT>), dim3((uint32_t)a.n * ntiles),
                     dim3(kSplitBlock), 0, stream, a, ntiles);
  hipLaunchKernelGGL((rows_topp_finish_kernel<T, VEC>), dim3(a.n), dim3(kHistBlock), 0, stream, a,
                     ntiles);
  return hipGetLastError();
}

}  // namespace

bool topp_supported(const RowArgs& a) {
  const int64_t groups = (a.vocab + 3) >> 2;
  const int64_t tiles = (groups + kDrawTile - 1) / kDrawTile;
  return a.topp_rows != nullptr && a.topp_list != nullptr && a.split_partials != nullptr &&
         tiles <= kMaxSplit && (int64_t)a.n * tiles < 0x7FFFFFFF;
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
