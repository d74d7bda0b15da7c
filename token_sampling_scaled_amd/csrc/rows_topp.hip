// Top-p route (every row of the call filtered by top-p only, or unfiltered):
// three kernels; the row is read once by each of the first two.
//
// 1. rows_topp_hist_kernel, one workgroup of 1024 threads per row.  With
//    s2 = x log2(e) / T, every entry above -inf weighs exp2(s2 - m0), where the
//    reference m0 is the largest s2 of the first 4-entry group of every thread
//    (loaded alone, before the rest of the row, so that the wait for it is
//    short).
//    - A histogram over kBuckets equal buckets of s2 in [top2 - span, top2],
//      counted from the top: top2 = m0 + kHeadroom and span = kHeadroom + 1 +
//      max(0, log2(V / (1 - p))).  The entries below that range weigh less
//      than (1 - p) Z all together (Z, the row's mass, is at least that of the
//      row maximum, which lies within kHeadroom of m0), so the top-p cutoff
//      lies inside it.  Every entry adds a fixed-point mass relative to an
//      edge, 2^20 exp2(-(position - edge) w) rounded, with a 64-bit
//      integer LDS atomic, so the sums do not depend on the order of the
//      atomics: in-range entries to their bucket (edge: its upper end), the
//      entries below the range to a spare slot of their lane (edge: the
//      range's lower end).  A unit of a bucket weighs 2^-20 exp2(edge - m0).
//    - The first nonempty bucket from the top whose cumulative mass reaches
//      p Z holds the cutoff tie group: bucket b*.  Its entries are exactly
//      those with x_lo <= x < x_hi, and those above it have x >= x_hi: both
//      bounds are the smallest order keys past a boundary of the same
//      (monotone) bucket function, found around a computed guess.
//    A row whose maximum lies above top2 repeats the pass with m0 = its
//    maximum.  Greedy rows and rows with no entry above -inf finish here.
// 2. rows_topp_draw_kernel, one 256-thread workgroup per (row, tile) item,
//    many more than the device holds at once: entries with x >= x_hi are
//    members of P; each wave queues its 4-entry groups holding a member and
//    draws one Philox block per queued group, 64 at a time.  Entries of b*
//    are appended (order key, index) to the row's list.  Each wave's best
//    member goes into the row's best with one 64-bit atomic maximum.
// 3. rows_topp_finish_kernel, one workgroup per row: the exact cutoff tie
//    group inside b* from the list -- the largest key v whose entries at or
//    above v, with the mass above b*, reach p Z, so whole tie groups stay
//    together -- the noise of the list's members of P, the best of them and
//    of the draw, the id and its log-prob.  A list that overflowed its
//    capacity is rebuilt from the row by radix passes over the order keys.
#include "split_common.hpp"

namespace tss {

namespace {

using namespace split;

constexpr int kHistBlock = 1024;
constexpr int kHistWaves = kHistBlock / kWave;
constexpr int kBuckets = 16384;
constexpr int kBucketsPerThread = kBuckets / kHistBlock;
constexpr float kHeadroom = 12.0f;    // base-2 units of s2 above m0 covered by the histogram
constexpr int kRing = 16;             // groups per thread in flight in the histogram pass
constexpr float kUnitLog2 = 20.0f;    // a mass relative to its bucket edge is held in units of 2^-20
constexpr float kMostNegative = -3.40282347e38f;
constexpr int kDrawBlock = 256;
constexpr int kDrawWaves = kDrawBlock / kWave;
constexpr int kDrawPT = 8;           // 4-entry groups per thread in a draw tile
constexpr int kDrawTile = kDrawPT * kDrawBlock;
constexpr int kQueue = 2 * kWave;     // queued member groups per wave
constexpr int kFinBlock = kTopPListCap;   // one list entry per thread
constexpr int kFinWaves = kFinBlock / kWave;
constexpr int kRadixBins = 2048;

template <typename T>
struct KeyRaw;
template <>
struct KeyRaw<float> {
  static constexpr uint32_t kLo = 0x00800000u;   // key of the most negative finite value
  static constexpr uint32_t kHi = 0xFF800000u;   // key of +inf
  __device__ __forceinline__ static float value_of_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  }
  __device__ __forceinline__ static uint32_t key_near(float x) {   // the key of x itself
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
};
template <>
struct KeyRaw<uint16_t> {
  static constexpr uint32_t kLo = 0x0080u;
  static constexpr uint32_t kHi = 0xFF80u;
  __device__ __forceinline__ static float value_of_key(uint32_t k) {
    const uint32_t raw = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    return __uint_as_float(raw << 16);
  }
  __device__ __forceinline__ static uint32_t key_near(float x) {   // x truncated to bf16
    const uint32_t u = __float_as_uint(x) >> 16;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
  }
};

// Scaled logit s2 = x log2(e) / T; NaN reads as -inf (the maximum of NaN and
// -inf is -inf).  A rounded product, so every kernel gets the same bits.
__device__ __forceinline__ float scaled2(float x, float scale2) {
  return fmaxf(__fmul_rn(x, scale2), -__builtin_inff());
}

// Position of a scaled logit in the histogram, (top2 - s2) inv_w, as one
// fused multiply-add from c = top2 inv_w: bucket floor(pos) when
// 0 <= pos < kBuckets, above the range when pos < 0, below it otherwise.
__device__ __forceinline__ float hist_pos(float s2, float inv_w, float c) {
  return __builtin_fmaf(s2, -inv_w, c);
}

__device__ __forceinline__ int bucket_of_pos(float pos) {
  return pos < 0.0f ? -1 : (pos < (float)kBuckets ? (int)pos : kBuckets);
}

// exp2 argument of an entry's fixed-point mass relative to its bucket's upper
// edge: 2^20 exp2(-(pos - floor(pos)) w) lies in [2^20 2^-w, 2^20].
__device__ __forceinline__ float unit_arg(float pos, float w) {
  return __builtin_fmaf(-__builtin_amdgcn_fractf(pos), w, kUnitLog2);
}

__device__ __forceinline__ uint32_t unit_round(float ex) { return (uint32_t)(ex + 0.5f); }

__device__ __forceinline__ uint32_t unit_mass(float pos, float w) {
  return unit_round(__builtin_amdgcn_exp2f(unit_arg(pos, w)));
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

__device__ __forceinline__ double wave_sum_f64(double v) {
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

// Bucket b lives in slot b + b/16 (one unused slot after every 16): the walk
// over the histogram after the pass, where thread t takes buckets 16t ..
// 16t + 15 in order, then reads slots 17t + j, which lie in distinct LDS banks
// across a wave; slots 16t + j would all share one bank pair.
constexpr int kHistSlots = kBuckets + kBuckets / 16;
constexpr int kHistAll = kHistSlots + kWave + kWave / 16;   // then the lanes' spare slots
__device__ __forceinline__ uint32_t hist_slot(uint32_t b) { return b + (b >> 4); }

struct HistShared {
  unsigned long long h64[kHistAll];   // the buckets, then the lanes' spare slots
  unsigned long long zb_units;        // the spare slots' sum
  double wscan[kHistWaves];
  float wmax[kHistWaves];
  uint32_t wkey[kHistWaves];
  int32_t wj[kHistWaves];
  int32_t hit;
  int32_t first;
  int32_t last;
  double hit_above, hit_scale;
};

template <typename T, bool VEC, int MODE>
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

  // the thread's first group goes out before the request's parameters are
  // read; it alone fixes the mass reference, so that the wait for it is short
  // (the ring of later loads is issued only after that)
  uint32_t ring[kRing][4];
  load_group<T, VEC>(row, v, groups, tid, ring[0]);

  const float temp = a.temperature[q];
  const float p = a.top_p ? a.top_p[q] : 1.0f;
  const bool greedy = !(temp >= 1e-5f);
  const uint64_t seed = a.seed[q];
  const uint64_t off = noise_offset(a, q);
  TopPRow* st = a.topp_rows + r;

  auto first_max = [&](bool nan_lp) {
    // first index of the largest order key (NaN as -inf, -0 as +0): greedy
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
    for (int off2 = 32; off2 > 0; off2 >>= 1) {
      const uint32_t ok = (uint32_t)__shfl_xor((int)bkey, off2, kWave);
      const int32_t oj = __shfl_xor(bj, off2, kWave);
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
      for (int w2 = 1; w2 < kHistWaves; ++w2) {
        if (sh.wkey[w2] > bkey || (sh.wkey[w2] == bkey && sh.wj[w2] < bj)) {
          bkey = sh.wkey[w2];
          bj = sh.wj[w2];
        }
      }
      const bool none = bj == 0x7FFFFFFF;
      if (MODE == kOutSample) {
        a.out_ids[r] = none ? -1 : bj;
        if (a.out_lp) a.out_lp[r] = (none || nan_lp) ? __builtin_nanf("") : 0.0f;
      } else {                   // log-probs: 0 at the greedy id, or a NaN row
        st->done_id = (none || nan_lp) ? -1 : bj;
      }
      st->mode = kTopPDone;
    }
  };
  if (greedy) {
    first_max(false);
    return;
  }

  const float scale2 = 1.4426950408889634f / temp;
  const bool p_on = p < 1.0f - 1e-6f;
  // histogram range below top2, in base-2 units: always the headroom and one
  // more, so the row maximum lies inside it
  const float span = kHeadroom + 1.0f +
                     fmaxf(__builtin_amdgcn_logf((float)v / fmaxf(1.0f - p, 1e-30f)), 0.0f);
  const float inv_w = (float)kBuckets / span;
  const float w = 1.0f / inv_w;

  // ---- mass reference: the largest s2 of the first group of every thread
  for (int s = tid; s < kHistAll; s += kHistBlock) sh.h64[s] = 0ull;
  float tmax = -__builtin_inff();
  if (tid < groups) {
#pragma unroll
    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, scaled2(E::value(ring[0][e]), scale2));
  }
  tmax = wave_max_f(tmax);
  if (lane == 0) sh.wmax[wid] = tmax;
  __syncthreads();
  float m0 = sh.wmax[0];
  for (int w2 = 1; w2 < kHistWaves; ++w2) m0 = fmaxf(m0, sh.wmax[w2]);
#pragma unroll
  for (int u = 1; u < kRing; ++u) load_group<T, VEC>(row, v, groups, tid + u * kHistBlock, ring[u]);

  // ---- the pass: every entry adds a fixed-point mass relative to an edge,
  // 2^20 exp2(-(pos - edge) w): in-range entries to their bucket (edge =
  // floor(pos)), the entries below the range to their lane's spare slot (edge
  // = kBuckets, the range's lower end; lanes hit distinct banks there).  An
  // entry just above top2 may land in bucket 0 and the ones further above in
  // a spare slot: the row is redone then anyway.
  float top2 = m0 + kHeadroom;
  float c = top2 * inv_w;
  const uint32_t spare = (uint32_t)(kBuckets + lane);
  auto add_group = [&](const uint32_t (&raw)[4]) {
    float s2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s2[e] = scaled2(E::value(raw[e]), scale2);
    tmax = fmaxf(tmax, fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3])));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pos = hist_pos(s2[e], inv_w, c);
      const int bi = (int)pos;
      const bool in = (uint32_t)bi < (uint32_t)kBuckets;
      const float rel = in ? __builtin_amdgcn_fractf(pos) : pos - (float)kBuckets;
      const uint32_t um = unit_round(__builtin_amdgcn_exp2f(__builtin_fmaf(-rel, w, kUnitLog2)));
      atomicAdd(&sh.h64[hist_slot(in ? (uint32_t)bi : spare)], (unsigned long long)um);
    }
  };
  auto row_max = [&]() {
    const float mw = wave_max_f(tmax);
    __syncthreads();   // every earlier reader of the wave slots is done; the atomics are
    if (lane == 0) sh.wmax[wid] = mw;
    __syncthreads();
    float mr = sh.wmax[0];
    for (int w2 = 1; w2 < kHistWaves; ++w2) mr = fmaxf(mr, sh.wmax[w2]);
    return mr;
  };
  // (with VEC every load is issued, a slot past the row re-reading its last
  // group, so the number of loads in flight is the same at every step)
  for (int32_t g0 = tid; g0 < groups; g0 += kRing * kHistBlock) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int32_t g = g0 + u * kHistBlock;
      if (g < groups) add_group(ring[u]);
      const int32_t gn = g + kRing * kHistBlock;
      if (VEC || gn < groups) load_group<T, VEC>(row, v, groups, gn, ring[u]);
    }
  }
  float mrow = row_max();
  if (mrow == -__builtin_inff()) {            // no entry above -inf
    if (tid == 0) {
      if (MODE == kOutSample) {
        a.out_ids[r] = -1;
        if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
      } else {
        st->done_id = -1;
      }
      st->mode = kTopPDone;
    }
    return;
  }
  if (mrow == __builtin_inff()) {             // +inf in the row: the first one, lp NaN
    first_max(true);
    return;
  }
  if (hist_pos(mrow, inv_w, c) < 0.0f) {
    // the maximum lies more than the headroom above m0 (pos is monotone in
    // s2, so no other entry lies above top2 unless it does): the pass again
    // with m0 = the row maximum (re-read from the caches)
    m0 = mrow;
    top2 = m0 + kHeadroom;
    c = top2 * inv_w;
    for (int s = tid; s < kHistAll; s += kHistBlock) sh.h64[s] = 0ull;
    __syncthreads();
    for_row_groups<T, VEC, kHistBlock>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
      add_group(raw);
    });
    (void)row_max();
  }

  // ---- bucket masses.  A unit of bucket b's fixed-point sum weighs
  // 2^-20 exp2(e_b - m0), e_b = (c - b) / inv_w its upper edge.  Thread t
  // owns buckets 16t + j, j = 0 .. 15: bucket 16t + j weighs exp2(-j / inv_w)
  // times bucket 16t (small arguments: single precision holds them to an
  // ulp), and bucket 16t's exponent D - 16t / inv_w, D = c / inv_w - m0, is
  // assembled from exact single-precision pieces (fma residuals and a
  // two-sum) and split into an integer and a fraction before the exp2.
  auto edge_weight = [&](int b) -> double {     // 2^-20 exp2(e_b - m0)
    const float res = __builtin_fmaf(-w, inv_w, 1.0f);   // 1 / inv_w = w (1 + res + ...)
    const float w_lo = w * res;
    const float cw = c * w;
    const float cw_lo = __builtin_fmaf(c, w, -cw);
    const float d_hi = cw - m0;                  // two-sum of cw and -m0
    const float bb = d_hi - cw;
    const float d_lo = ((cw - (d_hi - bb)) + (-m0 - bb)) + cw_lo + c * w_lo;
    const float fb = (float)b;
    const float p_hi = fb * w;
    const float p_lo = __builtin_fmaf(fb, w, -p_hi) + fb * w_lo;
    const float x_hi = d_hi - p_hi;              // two-sum of d_hi and -p_hi
    const float bb2 = x_hi - d_hi;
    const float x_lo = ((d_hi - (x_hi - bb2)) + (-p_hi - bb2)) + (d_lo - p_lo);
    const float n = __builtin_floorf(x_hi);
    const float f = (x_hi - n) + x_lo;
    return __builtin_ldexp((double)__builtin_amdgcn_exp2f(f), (int)n - (int)kUnitLog2);
  };
  const int b0 = tid * kBucketsPerThread;
  const double base = edge_weight(b0);          // per-unit weight of bucket b0
  if (wid == 0) {                               // the spare slots: the entries below the range
    const unsigned long long zu = wave_sum_u64(sh.h64[hist_slot((uint32_t)spare)]);
    if (lane == 0) sh.zb_units = zu;
  }
  // exp2(-j / inv_w), j = 0 .. 15, one per lane, read back as scalars
  const float ej_lane = __builtin_amdgcn_exp2f(-(float)(lane & (kBucketsPerThread - 1)) * w);
  // mass of bucket b0 + j relative to `base` (the same arithmetic wherever it
  // is needed, from the histogram in LDS)
  auto rel_mass = [&](int j) -> float {
    const unsigned long long h = sh.h64[hist_slot((uint32_t)(b0 + j))];
    const float hf = __builtin_fmaf((float)(uint32_t)(h >> 32), 4294967296.0f, (float)(uint32_t)h);
    return hf * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ej_lane), j));
  };
  double mine = 0.0;
  int firstne = 0x7FFFFFFF, lastne = -1;
#pragma unroll
  for (int j = 0; j < kBucketsPerThread; ++j) {
    const float mj = rel_mass(j);
    mine += (double)mj;
    if (mj != 0.0f) {
      firstne = min(firstne, b0 + j);
      lastne = b0 + j;
    }
  }
  mine *= base;
  // block scan of the thread masses: thread t's interval [excl, incl] ends
  // exactly where thread t + 1's begins
  double incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  if (lane == kWave - 1) sh.wscan[wid] = incl;
  if (tid == 0) {
    sh.hit = -1;
    sh.first = 0x7FFFFFFF;
    sh.last = -1;
  }
  __syncthreads();
  {
    // buckets rise with the thread: the wave's first nonempty bucket is its
    // first such lane's, the last one its last such lane's (one atomic each
    // per wave; a shared address takes its atomics one at a time)
    const unsigned long long ne = __ballot(lastne >= 0);
    if (ne) {
      if (lane == __builtin_ctzll(ne)) atomicMin(&sh.first, firstne);
      if (lane == 63 - __builtin_clzll(ne)) atomicMax(&sh.last, lastne);
    }
  }
  double pre = 0.0, zin = 0.0;
  for (int w2 = 0; w2 < kHistWaves; ++w2) {
    if (w2 == wid) pre = zin;
    zin += sh.wscan[w2];
  }
  excl += pre;
  incl += pre;
  const double zbelow = (double)sh.zb_units * edge_weight(kBuckets);
  if (!p_on) {                                  // P = every entry above -inf (uniform)
    if (tid == 0) {
      st->mode = kTopPAll;
      st->best = 0ull;
      st->inv_t = 1.0f / temp;
      st->x_hi = kMostNegative;
      st->x_lo = kMostNegative;
      st->m0 = m0;
      st->scale2 = scale2;
      st->nlist = 0;
      st->above = zin + zbelow;
      st->src = src;
      st->seed = seed;
      st->off = off;
    }
    return;
  }
  const double target = (double)p * (zin + zbelow);
  // the bucket b0 + j of this thread at cumulative mass `cj` when the walk
  // reaches it (the walk adds the buckets in the order of the sum above)
  auto walk_to = [&](int jstop, double& cj) {
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kBucketsPerThread; ++j)
      if (j < jstop) acc += (double)rel_mass(j);
    cj = excl + acc * base;
  };
  auto publish = [&](int b, double above_b) {
    sh.hit = b;
    sh.hit_above = above_b;
    sh.hit_scale = base * (double)__builtin_amdgcn_exp2f(-(float)(b - b0) * w);
  };
  if (excl < target && target <= incl) {
    // the first bucket of this thread whose cumulative mass reaches the
    // target; rounding may leave it unreached, then the last nonempty one
    double acc = 0.0;
    int hit = -1;
    double hit_above = 0.0;
#pragma unroll
    for (int j = 0; j < kBucketsPerThread; ++j) {
      const double cj = excl + acc * base;
      const float mj = rel_mass(j);
      acc += (double)mj;
      if (mj != 0.0f && hit < 0 && excl + acc * base >= target) {
        hit = b0 + j;
        hit_above = cj;
      }
    }
    if (hit < 0) {
      hit = lastne;
      walk_to(lastne - b0, hit_above);
    }
    publish(hit, hit_above);
  }
  __syncthreads();
  if (sh.hit < 0) {                             // uniform: the target lies outside the range's mass
    const bool low = target <= 0.0;
    const int bsel = low ? sh.first : sh.last;
    if (bsel >= b0 && bsel < b0 + kBucketsPerThread) {
      double cj = 0.0;
      if (!low) walk_to(bsel - b0, cj);
      publish(bsel, cj);
    }
    __syncthreads();
  }

  // ---- the bounds of b*'s entries: lanes 0 .. 31 look for the smallest key
  // whose bucket lies above b*, lanes 32 .. 63 for the smallest one whose
  // bucket is b* or above.  The bucket of a key's value never rises with the
  // key, and +inf lies above every bucket.  The boundary value of s2 is
  // about (c - lim - 1) / inv_w; the 32 keys around that guess are checked at
  // once, and a binary search over every key runs only if they miss it.
  if (wid == 0) {
    const int bstar = sh.hit < 0 ? 0 : sh.hit;
    const int half = lane >> 5;
    const int lim = half == 0 ? bstar - 1 : bstar;
    auto pred = [&](uint32_t key) {
      return bucket_of_pos(hist_pos(scaled2(KeyRaw<T>::value_of_key(key), scale2), inv_w, c)) <= lim;
    };
    const float xg = ((c - (float)(lim + 1)) * w) / scale2;
    const uint32_t kg = KeyRaw<T>::key_near(xg);
    const uint32_t k0 = kg < KeyRaw<T>::kLo + 16u ? KeyRaw<T>::kLo
                      : (kg > KeyRaw<T>::kHi - 15u ? KeyRaw<T>::kHi - 31u : kg - 16u);
    const uint32_t cand = k0 + (uint32_t)(lane & 31);
    const unsigned long long bal = __ballot(pred(cand));
    const uint32_t hb = (uint32_t)(bal >> (half * 32));
    uint32_t key;
    // found when the window holds the first true key: some are true, and
    // the first is not the window's first unless that is the smallest key
    const bool found = hb != 0u && ((hb & 1u) == 0u || k0 == KeyRaw<T>::kLo);
    if (found) {
      key = k0 + (uint32_t)__builtin_ctz(hb);
    } else {
      uint32_t lo = KeyRaw<T>::kLo, hi = KeyRaw<T>::kHi;
      while (lo < hi) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (pred(mid)) hi = mid;
        else lo = mid + 1;
      }
      key = lo;
    }
    const float bound = KeyRaw<T>::value_of_key(key);
    const float xb_hi = __shfl(bound, 0, kWave);
    const float xb_lo = __shfl(bound, 32, kWave);
    if (lane == 0) {
      st->mode = kTopPCut;
      st->best = 0ull;
      st->inv_t = 1.0f / temp;
      st->bstar = bstar;
      st->x_hi = xb_hi;
      st->x_lo = xb_lo;
      st->m0 = m0;
      st->scale2 = scale2;
      st->inv_w = inv_w;
      st->c = c;
      st->w = w;
      st->nlist = 0;
      st->above = sh.hit_above;
      st->target = target;
      st->bscale = sh.hit_scale;
      st->src = src;
      st->seed = seed;
      st->off = off;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. draw

// One workgroup per (row, tile) item (item = tile * n + r, so that the rows'
// tiles interleave), many more items than the device holds at once: the
// hardware deals them out as workgroups finish, which keeps the compute units
// evenly loaded however unevenly the members of P fall over the rows.  The
// tile's loads go out first.  Entries with x >= x_hi are members of P: each
// wave queues its groups holding a member in LDS and draws one Philox block
// per queued group, 64 at a time.  Entries of the cutoff bucket (x_lo <= x <
// x_hi) are appended to the row's list, one atomic per wave for its slots.
// Each wave's best member goes into the row's best with one 64-bit atomic
// maximum of (order of z2, complement of its index).
// With LP (log-prob calls) only the cutoff bucket's entries are listed, for
// the rows that have one.
template <typename T, bool VEC, bool LP>
__global__ __launch_bounds__(kDrawBlock) void rows_topp_draw_kernel(RowArgs a, int32_t ntiles) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ uint32_t qg[kDrawWaves][kQueue];        // queued groups
  __shared__ uint32_t qraw[kDrawWaves][kQueue][4];   // their raw entries

  const int r = (int)(blockIdx.x % (uint32_t)a.n);
  const int tile = (int)(blockIdx.x / (uint32_t)a.n);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  const int32_t t0 = tile * kDrawTile;
  const int32_t t_end = t0 + kDrawTile < groups ? t0 + kDrawTile : groups;
  const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
  const T* row = reinterpret_cast<const T*>(a.logits) + src * a.row_stride;
  // the row's state through the constant address space: scalar loads
  // (nothing this kernel writes is read this way).  Its mode first: a row
  // already finished (greedy, +inf, nothing finite) is not read at all.
  const __attribute__((address_space(4))) TopPRow* st =
      (const __attribute__((address_space(4))) TopPRow*)(a.topp_rows + r);
  if (st->mode == kTopPDone) return;             // uniform over the workgroup
  if (LP && st->mode != kTopPCut) return;

  uint32_t raw[kDrawPT][4];
#pragma unroll
  for (int i = 0; i < kDrawPT; ++i) load_group<T, VEC>(row, v, t_end, t0 + tid + i * kDrawBlock, raw[i]);

  const float x_hi = st->x_hi;
  const float x_lo = st->x_lo;
  const float scale2 = st->scale2;
  const uint64_t seed = st->seed;
  const uint64_t off = st->off;
  const NoiseStream ns{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r, (uint32_t)off,
                       (uint32_t)(off >> 32)};

  float bz = -__builtin_inff();                  // this lane's best member: z2, index
  int32_t bj = 0x7FFFFFFF;
  uint32_t fill = 0;                             // queued groups of this wave (uniform)
  auto drain = [&](uint32_t count) {             // draw the first count (<= 64) queued groups
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((uint32_t)lane < count) {
      const uint32_t g = qg[wid][lane];
      const Philox4 wd = ns.block(g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = E::value(qraw[wid][lane][e]);
        if (!(x >= x_hi)) continue;
        // members are finite: x * scale2 needs no NaN guard
        const float z2 = x * scale2 + gumbel2_from_word(wd.v[e]);
        const int32_t j = (int32_t)(g * 4 + e);
        if (z2 > bz || (z2 == bz && j < bj)) {
          bz = z2;
          bj = j;
        }
      }
    }
  };
  unsigned long long bnd_any = 0ull;             // lanes with a cutoff-bucket entry
#pragma unroll
  for (int i = 0; i < kDrawPT; ++i) {
    const int32_t g = t0 + tid + i * kDrawBlock;
    // lane masks (scalar): groups holding a member, and groups holding an
    // entry of the cutoff bucket (x >= x_lo but not x >= x_hi)
    const unsigned long long valid = __ballot(g < t_end);
    unsigned long long memm = 0ull, bndm = 0ull;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = E::value(raw[i][e]);
      const unsigned long long hi = __ballot(x >= x_hi);
      memm |= hi;
      bndm |= __ballot(x >= x_lo) ^ hi;
    }
    memm &= valid;
    bnd_any |= bndm & valid;
    if (LP) continue;                            // no noise for log-probs
    if ((memm >> lane) & 1ull) {
      const uint32_t pos = fill + lane_rank_u64(memm);
      qg[wid][pos] = (uint32_t)g;
#pragma unroll
      for (int e = 0; e < 4; ++e) qraw[wid][pos][e] = raw[i][e];
    }
    fill += (uint32_t)__popcll(memm);
    if (fill >= (uint32_t)kWave) {               // a full round of 64 groups: draw it
      drain(kWave);
      fill -= kWave;
      uint32_t mg = 0, m4[4] = {0u, 0u, 0u, 0u};
      if ((uint32_t)lane < fill) {                // move the rest to the front
        mg = qg[wid][kWave + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) m4[e] = qraw[wid][kWave + lane][e];
      }
      __builtin_amdgcn_wave_barrier();
      if ((uint32_t)lane < fill) {
        qg[wid][lane] = mg;
#pragma unroll
        for (int e = 0; e < 4; ++e) qraw[wid][lane][e] = m4[e];
      }
    }
  }
  if (!LP && fill) drain(fill);

  // the cutoff bucket's entries (a few per row): one atomic per wave
  // reserves their slots in the row's list
  if (bnd_any) {
    uint32_t nb = 0;
    uint32_t bmask[kDrawPT];
#pragma unroll
    for (int i = 0; i < kDrawPT; ++i) {
      const int32_t g = t0 + tid + i * kDrawBlock;
      uint32_t bm = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = E::value(raw[i][e]);
        bm |= (g < t_end && x >= x_lo && !(x >= x_hi) ? 1u : 0u) << e;
      }
      bmask[i] = bm;
      nb += (uint32_t)__popc(bm);
    }
    uint32_t incl = nb;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_up((int)incl, o, kWave);
      if (lane >= o) incl += t;
    }
    uint32_t base = 0;
    if (lane == kWave - 1) base = atomicAdd(&a.topp_rows[r].nlist, incl);
    base = (uint32_t)__shfl((int)base, kWave - 1, kWave) + incl - nb;
    TopPCand* list = a.topp_list + (int64_t)r * kTopPListCap;
    // (static indexes only: an index into raw[] known only at run time
    // would put the whole tile in scratch memory)
#pragma unroll
    for (int i = 0; i < kDrawPT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((bmask[i] >> e) & 1u) {
          if (base < (uint32_t)kTopPListCap)
            list[base] = TopPCand{K::from_bits(raw[i][e]), (t0 + tid + i * kDrawBlock) * 4 + e};
          ++base;
        }
      }
    }
  }
  // the wave's best: the largest (order of z2, -index)
  unsigned long long key =
      bj == 0x7FFFFFFF ? 0ull
                       : ((unsigned long long)order_of(bz) << 32) | (unsigned long long)(~(uint32_t)bj);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long t = __shfl_xor(key, o, kWave);
    key = t > key ? t : key;
  }
  if (!LP && lane == 0 && key != 0ull) atomicMax(&a.topp_rows[r].best, key);
}

// ---------------------------------------------------------------------------
// 3. finish

struct FinShared {
  alignas(16) uint2 ent[kTopPListCap];   // the list: (order key, fixed-point mass)
  unsigned long long mass[kRadixBins];   // radix bins (overflow path)
  unsigned long long wtot[kFinWaves];
  double wz[kFinWaves];
  Best wbest[kFinWaves];
  uint32_t wkmin[kFinWaves];
  int32_t hit;
  int32_t first;
  int32_t last;
  unsigned long long hit_above;
  unsigned long long hit_mass;
};

// In bins [0, nb) ordered from the largest keys down, the first nonempty bin
// whose cumulative mass, on top of `base` units and the mass `above`,
// reaches `target` (the first nonempty bin when base already does; the last
// nonempty bin if none does).  Bin masses are fixed-point units worth `unit`
// each.  Writes the bin, the units above it and its own units to LDS (valid
// after the call in every thread).
__device__ __forceinline__ void find_crossing(FinShared& sh, int nb, unsigned long long base,
                                              double above, double unit, double target) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int per = nb / kFinBlock;
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
    if (m && above + (double)cum * unit < target && above + (double)(cum + m) * unit >= target) {
      sh.hit = b;
      sh.hit_above = cum - base;
      sh.hit_mass = m;
    }
    cum += m;
  }
  __syncthreads();
  if (above + (double)base * unit >= target) {
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
      for (int w = 0; w < kFinWaves; ++w) tot += sh.wtot[w];
      sh.hit = b;
      sh.hit_mass = b >= 0 ? sh.mass[b] : 0ull;
      sh.hit_above = tot - sh.hit_mass;
    }
    __syncthreads();
  }
}

// id and log-prob: lp = (s2 - m0 - log2(mass of P)) ln 2.
__device__ __forceinline__ void write_row(const RowArgs& a, int r, const Best& b, float m0,
                                          double zp) {
  if (b.j == 0x7FFFFFFF) {            // cannot happen: P holds the row maximum
    a.out_ids[r] = -1;
    if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
    return;
  }
  a.out_ids[r] = b.j;
  if (a.out_lp) a.out_lp[r] = (float)(((double)b.s - (double)m0 - log2(zp)) * 0.69314718055994531);
}

// Block-wide best (valid in thread 0).
__device__ __forceinline__ Best block_best(Best b, FinShared& sh) {
  b = wave_best(b);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sh.wbest[wid] = b;
  __syncthreads();
  Best o = sh.wbest[0];
  for (int w = 1; w < kFinWaves; ++w)
    if (beats(sh.wbest[w].o, sh.wbest[w].j, o.o, o.j)) o = sh.wbest[w];
  return o;
}

// Log-prob calls (thread 0): P = {x >= x_cut} of mass zp.  At ids the entry's
// log-prob now, (s2 - m0 - log2 zp) ln 2 as for a sampled id; full rows leave
// the cutoff to the write kernel.
template <typename T, int MODE>
__device__ __forceinline__ void lp_finish(const RowArgs& a, int r, TopPRow* st, float x_cut,
                                          double zp) {
  using E = SplitElem<T>;
  if (MODE == kOutLogProbAt) {
    const int64_t j = a.token_ids[r];
    float out = -__builtin_inff();
    if (j >= 0 && j < a.vocab) {
      const T* row = reinterpret_cast<const T*>(a.logits) + st->src * a.row_stride;
      const float x = E::value(E::raw_at(row, j));
      if (x >= x_cut)
        out = (float)(((double)scaled2(x, st->scale2) - (double)st->m0 - log2(zp)) * 0.69314718055994531);
    }
    a.out_lp[r] = out;
  } else {
    st->x_cut = x_cut;
    st->zp = zp;
  }
}

template <typename T, bool VEC, int MODE>
__global__ __launch_bounds__(kFinBlock) void rows_topp_finish_kernel(RowArgs a) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ FinShared sh;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;

  // the row's state and its whole list capacity are read at once
  TopPRow* st = a.topp_rows + r;
  const TopPCand mine_c = a.topp_list[(int64_t)r * kTopPListCap + tid];
  const uint32_t mode = st->mode;
  if (mode == kTopPDone) {
    if (MODE == kOutLogProbAt && tid == 0) {    // 0 at the greedy id, or NaN
      const int32_t id = st->done_id;
      const int64_t j = a.token_ids[r];
      a.out_lp[r] = id < 0 ? __builtin_nanf("") : (j == id ? 0.0f : -__builtin_inff());
    }
    return;
  }
  const float m0 = st->m0;
  if (MODE != kOutSample && mode == kTopPAll) {
    if (tid == 0) lp_finish<T, MODE>(a, r, st, kMostNegative, st->above);
    return;
  }
  // the draw's best member (thread 0): its order word, its index, and its
  // scaled logit read back from the row
  Best tb{0u, 0x7FFFFFFF, 0.0f};
  if (tid == 0 && st->best != 0ull) {
    const unsigned long long bk = st->best;
    const int32_t j = (int32_t)~(uint32_t)bk;
    const T* brow = reinterpret_cast<const T*>(a.logits) + st->src * a.row_stride;
    tb = Best{(uint32_t)(bk >> 32), j, scaled2(E::value(E::raw_at(brow, j)), st->scale2)};
  }
  if (mode == kTopPAll) {
    tb = block_best(tb, sh);
    if (tid == 0) write_row(a, r, tb, m0, st->above);
    return;
  }
  const uint32_t nlist = st->nlist;
  const float scale2 = st->scale2;
  const float inv_w = st->inv_w;
  const float c = st->c;
  const float w = st->w;
  const double above = st->above;
  const double target = st->target;
  const double bscale = st->bscale;
  const NoiseStream ns{(uint32_t)st->seed, (uint32_t)(st->seed >> 32), (uint32_t)r,
                       (uint32_t)st->off, (uint32_t)(st->off >> 32)};

  if (nlist <= (uint32_t)kTopPListCap) {
    // ---- the list holds every entry of b*: entry i is in P when the mass
    // above b* plus that of the list's entries with a strictly larger key
    // stays below the target (whole tie groups together); the row's top
    // group is always kept
    const bool in = (uint32_t)tid < nlist;
    float s2 = 0.0f;
    uint32_t um = 0;
    if (in) {
      s2 = scaled2(KeyRaw<T>::value_of_key(mine_c.key), scale2);
      um = unit_mass(hist_pos(s2, inv_w, c), w);
    }
    sh.ent[tid] = make_uint2(in ? mine_c.key : 0u, um);   // slots past the list weigh 0
    __syncthreads();
    unsigned long long gt = 0;
    if (in) {
      // eight entries per step, read as 16-byte words
      const uint4* e4 = reinterpret_cast<const uint4*>(sh.ent);
      for (uint32_t t = 0; t < nlist; t += 8) {
        uint4 q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = e4[(t >> 1) + i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gt += q[i].x > mine_c.key ? (unsigned long long)q[i].y : 0ull;
          gt += q[i].z > mine_c.key ? (unsigned long long)q[i].w : 0ull;
        }
      }
    }
    const bool keep = in && (above + (double)gt * bscale < target || (above == 0.0 && gt == 0));
    double zw = keep ? (double)um * bscale : 0.0;
    if (MODE != kOutSample) {
      // P = everything above b* and the kept top of b*: x >= the smallest
      // kept value (canonical keys: -0 goes with +0)
      uint32_t kmin = keep ? mine_c.key : 0xFFFFFFFFu;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, kWave));
      zw = wave_sum_f64(zw);
      if (lane == 0) {
        sh.wz[wid] = zw;
        sh.wkmin[wid] = kmin;
      }
      __syncthreads();
      if (tid == 0) {
        double zp = above;
        uint32_t km = 0xFFFFFFFFu;
        for (int w2 = 0; w2 < kFinWaves; ++w2) {
          zp += sh.wz[w2];
          km = min(km, sh.wkmin[w2]);
        }
        lp_finish<T, MODE>(a, r, st, km == 0xFFFFFFFFu ? st->x_hi : KeyRaw<T>::value_of_key(km), zp);
      }
      return;
    }
    Best lb = tb;
    if (keep) {
      const float z2 = s2 + gumbel2_from_word(ns.word((uint32_t)mine_c.j));
      const uint32_t o = order_of(z2);
      if (beats(o, mine_c.j, lb.o, lb.j)) lb = Best{o, mine_c.j, s2};
    }
    zw = wave_sum_f64(zw);
    if (lane == 0) sh.wz[wid] = zw;
    lb = block_best(lb, sh);
    if (tid == 0) {
      double zp = above;
      for (int w2 = 0; w2 < kFinWaves; ++w2) zp += sh.wz[w2];
      write_row(a, r, lb, m0, zp);
    }
    return;
  }

  // ---- overflow: radix passes over the order keys of b*'s entries read from
  // the row, on the cumulative mass, then the noise of b*'s members of P
  const float x_hi = st->x_hi;
  const float x_lo = st->x_lo;
  const T* row = reinterpret_cast<const T*>(a.logits) + st->src * a.row_stride;
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  uint32_t prefix = 0;
  unsigned long long base = 0, zp_units = 0;
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBits[3] = {11, 11, 10};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shf = kShift[pass], bits = kBits[pass];
    for (int b = tid; b < kRadixBins; b += kFinBlock) sh.mass[b] = 0;
    __syncthreads();
    for_row_groups<T, VEC, kFinBlock>(row, v, groups, [&](int32_t, const uint32_t (&raw)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = E::value(raw[e]);
        if (!(x >= x_lo && x < x_hi)) continue;
        const uint32_t key = K::from_bits(raw[e]);
        if (pass > 0 && (key >> (shf + bits)) != prefix) continue;
        const int d = (int)((key >> shf) & ((1u << bits) - 1u));
        atomicAdd(&sh.mass[(kRadixBins - 1) - d],
                  (unsigned long long)unit_mass(hist_pos(scaled2(x, scale2), inv_w, c), w));
      }
    });
    __syncthreads();
    find_crossing(sh, kRadixBins, base, above, bscale, target);
    const int d = (kRadixBins - 1) - (sh.hit < 0 ? 0 : sh.hit);
    base += sh.hit_above;
    prefix = (prefix << bits) | (uint32_t)d;
    zp_units = base + sh.hit_mass;
    __syncthreads();
  }
  const uint32_t vstar = prefix;
  if (MODE != kOutSample) {
    if (tid == 0)
      lp_finish<T, MODE>(a, r, st, KeyRaw<T>::value_of_key(vstar), above + (double)zp_units * bscale);
    return;
  }
  for_row_groups<T, VEC, kFinBlock>(row, v, groups, [&](int32_t g, const uint32_t (&raw)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = E::value(raw[e]);
      if (!(x >= x_lo && x < x_hi) || K::from_bits(raw[e]) < vstar) continue;
      const int32_t j = g * 4 + e;
      const float s2 = scaled2(x, scale2);
      const float z2 = s2 + gumbel2_from_word(ns.word((uint32_t)j));
      const uint32_t o = order_of(z2);
      if (beats(o, j, tb.o, tb.j)) tb = Best{o, j, s2};
    }
  });
  tb = block_best(tb, sh);
  if (tid == 0) write_row(a, r, tb, m0, above + (double)zp_units * bscale);
  (void)lane;
}

// ---------------------------------------------------------------------------
// 4. full-row log-probs: one 256-thread workgroup per (row, tile of 1024
// groups) writes lp = x / T - (m0 + log2 zp) ln 2 on P and -inf elsewhere
// (a greedy row: 0 at its id; a row with nothing finite: NaN).

constexpr int kWriteBlock = 256;
constexpr int kWritePT = 4;
constexpr int kWriteTile = kWritePT * kWriteBlock;

template <typename T, bool VEC>
__global__ __launch_bounds__(kWriteBlock) void rows_topp_lp_write_kernel(RowArgs a, int32_t ntiles) {
  using E = SplitElem<T>;
  const int r = (int)(blockIdx.x % (uint32_t)a.n);
  const int tile = (int)(blockIdx.x / (uint32_t)a.n);
  const int tid = threadIdx.x;
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  const int32_t t0 = tile * kWriteTile;
  const int32_t t_end = t0 + kWriteTile < groups ? t0 + kWriteTile : groups;
  const __attribute__((address_space(4))) TopPRow* st =
      (const __attribute__((address_space(4))) TopPRow*)(a.topp_rows + r);
  float* out = a.out_lp + (int64_t)r * v;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  if (st->mode == kTopPDone) {
    const int32_t id = st->done_id;
    for (int i = 0; i < kWritePT; ++i) {
      const int32_t g = t0 + tid + i * kWriteBlock;
      if (g >= t_end) break;
      for (int e = 0; e < 4 && (int64_t)g * 4 + e < v; ++e) {
        const int64_t j = (int64_t)g * 4 + e;
        out[j] = id < 0 ? __builtin_nanf("") : (j == id ? 0.0f : -__builtin_inff());
      }
    }
    return;
  }
  const int64_t src = st->src;
  const T* row = reinterpret_cast<const T*>(a.logits) + src * a.row_stride;
  uint32_t raw[kWritePT][4];
#pragma unroll
  for (int i = 0; i < kWritePT; ++i) load_group<T, VEC>(row, v, t_end, t0 + tid + i * kWriteBlock, raw[i]);
  const float x_cut = st->x_cut;
  const float inv_t = st->inv_t;
  const float c0 = (float)(((double)st->m0 + log2(st->zp)) * 0.69314718055994531);
#pragma unroll
  for (int i = 0; i < kWritePT; ++i) {
    const int32_t g = t0 + tid + i * kWriteBlock;
    if (g >= t_end) continue;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = E::value(raw[i][e]);
      o[e] = x >= x_cut ? __builtin_fmaf(x, inv_t, -c0) : -__builtin_inff();
    }
    if (VEC) {
      *reinterpret_cast<f32x4*>(out + (int64_t)g * 4) = f32x4{o[0], o[1], o[2], o[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((int64_t)g * 4 + e < v) out[(int64_t)g * 4 + e] = o[e];
    }
  }
}

template <typename T, bool VEC>
hipError_t launch_typed(const RowArgs& a, int32_t ntiles, hipStream_t stream) {
  hipLaunchKernelGGL((rows_topp_hist_kernel<T, VEC, kOutSample>), dim3(a.n), dim3(kHistBlock), 0, stream, a);
  hipLaunchKernelGGL((rows_topp_draw_kernel<T, VEC, false>), dim3((uint32_t)a.n * ntiles), dim3(kDrawBlock),
                     0, stream, a, ntiles);
  hipLaunchKernelGGL((rows_topp_finish_kernel<T, VEC, kOutSample>), dim3(a.n), dim3(kFinBlock), 0, stream, a);
  return hipGetLastError();
}

template <typename T, bool VEC, int MODE>
hipError_t launch_lp_typed(const RowArgs& a, int32_t ntiles, hipStream_t stream) {
  hipLaunchKernelGGL((rows_topp_hist_kernel<T, VEC, MODE>), dim3(a.n), dim3(kHistBlock), 0, stream, a);
  hipLaunchKernelGGL((rows_topp_draw_kernel<T, VEC, true>), dim3((uint32_t)a.n * ntiles), dim3(kDrawBlock),
                     0, stream, a, ntiles);
  hipLaunchKernelGGL((rows_topp_finish_kernel<T, VEC, MODE>), dim3(a.n), dim3(kFinBlock), 0, stream, a);
  if (MODE == kOutLogProbFull) {
    const int64_t groups = (a.vocab + 3) >> 2;
    const int64_t wt = (groups + kWriteTile - 1) / kWriteTile;
    hipLaunchKernelGGL((rows_topp_lp_write_kernel<T, VEC>), dim3((uint32_t)(a.n * wt)), dim3(kWriteBlock),
                       0, stream, a, (int32_t)wt);
  }
  return hipGetLastError();
}

}  // namespace

bool topp_supported(const RowArgs& a) {
  const int64_t groups = (a.vocab + 3) >> 2;
  const int64_t tiles = (groups + kDrawTile - 1) / kDrawTile;
  return a.topp_rows != nullptr && a.topp_list != nullptr && (int64_t)a.n * tiles < 0x7FFFFFFF;
}

hipError_t launch_rows_topp_lp(const RowArgs& a, DType dtype, OutMode mode, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int64_t groups = (a.vocab + 3) >> 2;
  const int32_t ntiles = (int32_t)((groups + kDrawTile - 1) / kDrawTile);
  const uintptr_t base = reinterpret_cast<uintptr_t>(a.logits);
  const bool full = mode == kOutLogProbFull;
  // the write pass stores four log-probs at a time (16 bytes)
  const bool out_vec = !full || (reinterpret_cast<uintptr_t>(a.out_lp) % 16) == 0;
  if (dtype == kF32) {
    const bool vec = (base % 16) == 0 && (a.row_stride % 4) == 0 && (a.vocab % 4) == 0 && out_vec;
    if (vec) return full ? launch_lp_typed<float, true, kOutLogProbFull>(a, ntiles, stream)
                         : launch_lp_typed<float, true, kOutLogProbAt>(a, ntiles, stream);
    return full ? launch_lp_typed<float, false, kOutLogProbFull>(a, ntiles, stream)
                : launch_lp_typed<float, false, kOutLogProbAt>(a, ntiles, stream);
  }
  const bool vec = (base % 8) == 0 && (a.row_stride % 4) == 0 && (a.vocab % 4) == 0 && out_vec;
  if (vec) return full ? launch_lp_typed<uint16_t, true, kOutLogProbFull>(a, ntiles, stream)
                       : launch_lp_typed<uint16_t, true, kOutLogProbAt>(a, ntiles, stream);
  return full ? launch_lp_typed<uint16_t, false, kOutLogProbFull>(a, ntiles, stream)
              : launch_lp_typed<uint16_t, false, kOutLogProbAt>(a, ntiles, stream);
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
