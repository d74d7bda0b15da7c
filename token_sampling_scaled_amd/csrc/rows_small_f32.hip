// Short fp32 rows with an active top-k ("core.inference.sampling.flashinfer_sampling",
// sample_kernel: top-k, then top-p inside K, then the perturbed argmax): one
// workgroup of 1024 threads per row, the whole row in registers (up to 8192
// entries, two 16-byte vectors per thread).
//
//  1. Order keys of the row (NaN read as -inf, -0 as +0) and a histogram of
//     their top 11 bits over the finite entries.
//  2. Suffix counts of the 2048 bins give the lowest bin b* whose bins at and
//     above it hold at least |K| = min(k, finite entries) entries.
//  3. Those entries (the candidates) go to shared memory, each candidate's rank
//     in the order (value descending, index ascending) is counted against all
//     the others, and the first |K| land sorted.
//  4. One wave: masses exp(x/T - m) of K in that order, the tie groups from the
//     top whose mass before them stays below p * Z_K (at least one), then
//     Philox noise for each member of P and the argmax of x/T + g; or, for
//     log-probs, the rank word of P's last member and ln Z_P, after which
//     every thread writes its own entries (full rows) or thread 0 the one at
//     the request's id.
//
// The ranking threads also weigh their members of K and draw their noise, so
// that wave 0 is left with two prefix sums and an argmax.  Rows the body does
// not take run the general per-row body in the same workgroup: greedy rows, k
// inactive or above 256, more than 1024 candidates, a +inf maximum, no finite
// entry.
#include "general_row.hpp"

namespace tss {

namespace {

constexpr int kB = 1024;
constexpr int kWv = kB / kWave;
constexpr int kNV = 2;                      // 16-byte vectors per thread
constexpr int kBins = 2048;                 // top 11 bits of a 32-bit order key
constexpr int kMaxK = 4 * kWave;            // K: four entries per lane of one wave
constexpr int kCandCap = kB;                // one candidate per thread when ranking
constexpr uint32_t kPosInfKey = 0xFF800000u;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// An entry's place in the order (value descending, index ascending) as one
// 64-bit word: order key above, complemented index below; larger is earlier.
__device__ __forceinline__ uint64_t rank_word(uint32_t key, int32_t j) {
  return ((uint64_t)key << 32) | (uint32_t)~j;
}

struct SmallShared {
  uint32_t hist[kBins];
  alignas(16) uint64_t cand[kCandCap + 8];   // candidates' rank words, zero padded to 8
  uint64_t sorted[kMaxK];           // K in the order: rank words ...
  float sw[kMaxK];                  // ... weights exp(x/T - m) ...
  float sz[kMaxK];                  // ... and perturbed scores x/T + g
  uint32_t wtot[kWv];
  uint32_t wmax[kWv];               // per-wave largest order key
  uint64_t lastw;                   // log-probs: rank word of P's last member ...
  float lzp;                        // ... and ln Z_P
  uint32_t nc;                      // candidates appended so far
  uint32_t bstar;                   // lowest candidate bin
  uint32_t ncand;                   // entries in the bins at and above it
};

union Shared {
  SmallShared s;
  general::Shared g;
};

__device__ __forceinline__ float value_of_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Step 4 (wave 0; lane l holds entries 4l .. 4l+3 of K): P inside K, then the
// draw (sampling), or the last member of P and ln Z_P for every thread
// (log-probs).
template <int ROUTE, int MODE>
__device__ __forceinline__ void draw_or_cut(const RowArgs& a, int r, SmallShared& sm, uint32_t kk,
                                            float pq, float inv_t, float m) {
  constexpr bool kHasP = ROUTE == kRouteJoint;
  const int lane = threadIdx.x & (kWave - 1);
  float x[4], w[4], zz[4], pre[4];
  int32_t jj[4];
  float lsum = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = 4u * lane + e;
    const uint64_t rw = i < kk ? sm.sorted[i] : 0ull;
    jj[e] = (int32_t)~(uint32_t)rw;
    x[e] = i < kk ? value_of_key((uint32_t)(rw >> 32)) : 0.0f;
    w[e] = i < kk ? sm.sw[i] : 0.0f;
    zz[e] = (MODE == kOutSample && i < kk) ? sm.sz[i] : -__builtin_inff();
    pre[e] = lsum;                   // mass of the entries before it, inside the lane
    lsum += w[e];
  }
  const float li = wave_scan_f32(lsum);
  const float zk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(li), kWave - 1));
  const float lex = li - lsum;
  // the first tie group (after the top one) whose mass before it reaches
  // p * Z_K starts the entries left out
  uint32_t cut = kk;
  if (kHasP && pq < 1.0f - 1e-6f) {
    const float xprev = __shfl_up(x[3], 1, kWave);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = 4u * lane + e;
      const float xp = e == 0 ? xprev : x[e - 1];
      const bool start = i > 0 && i < kk && x[e] != xp;
      if (start && (lex + pre[e]) / zk >= pq && i < cut) cut = i;
    }
    cut = wave_min_dpp(cut);
  }
  float zl = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) zl += (4u * lane + e < cut) ? w[e] : 0.0f;
  const float zp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_scan_f32(zl)), kWave - 1));
  if constexpr (MODE != kOutSample) {
    if (lane == 0) {
      sm.lastw = sm.sorted[cut - 1];
      sm.lzp = __logf(zp);
    }
    return;
  }

  ArgBest best{-__builtin_inff(), 0x7FFFFFFF};
  float sbest = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = 4u * lane + e;
    if (i < cut && better(zz[e], jj[e], best.z, best.j)) {
      best = ArgBest{zz[e], jj[e]};
      sbest = __fmul_rn(x[e], inv_t);
    }
  }
  // the largest score, the smallest index among equal ones
  const float zmax = wave_max_f32_dpp(best.z);
  const bool top = best.z == zmax;
  const uint32_t jmin = wave_min_dpp(top ? (uint32_t)best.j : 0xFFFFFFFFu);
  const unsigned long long own = __ballot(top && (uint32_t)best.j == jmin);
  const int sl = __ffsll((long long)own) - 1;
  const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sbest), sl));
  if (lane == 0) {
    a.out_ids[r] = (int32_t)jmin;
    if (a.out_lp) a.out_lp[r] = sw - m - __logf(zp);
  }
}

template <int ROUTE, int MODE>
__global__ __launch_bounds__(kB) void rows_small_f32_kernel(RowArgs a) {
  constexpr bool kHasP = ROUTE == kRouteJoint;
  __shared__ Shared sh;
  SmallShared& sm = sh.s;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
  const int64_t q = a.req_map ? (int64_t)a.req_map[r] : (int64_t)r;
  const int nvec = (int)(a.vocab >> 2);
  const f32x4* row = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.logits) +
                                                    src * a.row_stride);
  f32x4 d[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const int vi = i * kB + tid;
    d[i] = row[vi < nvec ? vi : nvec - 1];
  }
  const float temp = a.temperature[q];
  const int32_t kq = a.top_k[q];
  const float pq = kHasP ? a.top_p[q] : 1.0f;
  const uint64_t seed = a.seed[q];
  if (!(temp >= 1e-5f) || !(kq >= 1 && (int64_t)kq < a.vocab) || kq > kMaxK) {
    general::general_row<float, ROUTE, MODE>(a, r, sh.g);
    return;
  }

  // ---- 1. order keys and the histogram of their top 11 bits
  for (int i = tid; i < kBins; i += kB) sm.hist[i] = 0u;
  if (tid == 0) sm.nc = 0u;
  __syncthreads();
  uint32_t key[kNV][4];
  uint32_t kmx = 0;
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const bool in = i * kB + tid < nvec;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[i][e] = in ? KeyF32::from_bits(__float_as_uint(d[i][e])) : KeyF32::kNegInf;
      kmx = max(kmx, key[i][e]);
      if (key[i][e] > KeyF32::kNegInf) atomicAdd(&sm.hist[key[i][e] >> 21], 1u);
    }
  }
  kmx = wave_max_dpp(kmx);
  if (lane == 0) sm.wmax[wid] = kmx;
  __syncthreads();

  // ---- 2. thread t holds bins 2t and 2t + 1; the bin where the count from
  // the top reaches |K| is found by exactly one thread
  const uint32_t h0 = sm.hist[2 * tid], h1 = sm.hist[2 * tid + 1];
  const uint32_t c = h0 + h1;
  const uint32_t incl = wave_scan_u32(c);
  if (lane == kWave - 1) sm.wtot[wid] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
  kmx = 0;
#pragma unroll
  for (int w = 0; w < kWv; ++w) {
    const uint32_t t = sm.wtot[w];
    total += t;
    if (w < wid) before += t;
    kmx = max(kmx, sm.wmax[w]);
  }
  if (total == 0 || kmx >= kPosInfKey) {   // no finite entry, or a +inf
    __syncthreads();
    general::general_row<float, ROUTE, MODE>(a, r, sh.g);
    return;
  }
  const uint32_t kk = min((uint32_t)kq, total);   // |K|
  const uint32_t above = total - (before + incl);  // bins above 2t + 1
  if (above < kk && above + c >= kk) {
    const bool hi = above + h1 >= kk;
    sm.bstar = hi ? 2u * tid + 1u : 2u * tid;
    sm.ncand = hi ? above + h1 : above + c;
  }
  __syncthreads();
  const uint32_t bstar = sm.bstar;
  const uint32_t ncand = sm.ncand;
  if (ncand > (uint32_t)kCandCap) {
    __syncthreads();
    general::general_row<float, ROUTE, MODE>(a, r, sh.g);
    return;
  }

  // ---- 3. candidates to shared memory, then their ranks
  {
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < kNV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += (key[i][e] > KeyF32::kNegInf && (key[i][e] >> 21) >= bstar) ? 1u : 0u;
    const uint32_t wi = wave_scan_u32(cnt);
    uint32_t base = 0;
    if (lane == kWave - 1 && wi != 0) base = atomicAdd(&sm.nc, wi);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
    uint32_t pos = base + wi - cnt;
#pragma unroll
    for (int i = 0; i < kNV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[i][e] > KeyF32::kNegInf && (key[i][e] >> 21) >= bstar)
          sm.cand[pos++] = rank_word(key[i][e], (i * kB + tid) * 4 + e);
    // zeros up to a multiple of 8 words (no candidate's word is 0: its key is
    // above that of -inf)
    if ((uint32_t)tid >= ncand && (uint32_t)tid < ((ncand + 7u) & ~7u)) sm.cand[tid] = 0ull;
  }
  __syncthreads();
  // the row maximum x_max: m = x_max / T; each member of K gets its weight and
  // its perturbed score from the thread that ranked it
  const float inv_t = 1.0f / temp;
  const float m = __fmul_rn(value_of_key(kmx), inv_t);
  const uint64_t off = noise_offset(a, q);
  const NoiseStream nst{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r, (uint32_t)off,
                        (uint32_t)(off >> 32)};
  if ((uint32_t)tid < ncand) {
    // rank = the number of candidates earlier in the order; eight words per
    // step, four 16-byte reads in flight
    const uint64_t mine = sm.cand[tid];
    const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(sm.cand);
    uint32_t rank = 0;
    for (uint32_t o = 0; o < ncand; o += 8) {
      ulonglong2 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = c2[o / 2 + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) rank += (w[u].x > mine ? 1u : 0u) + (w[u].y > mine ? 1u : 0u);
    }
    if (rank < kk) {
      const float sv = __fmul_rn(value_of_key((uint32_t)(mine >> 32)), inv_t);
      sm.sorted[rank] = mine;
      sm.sw[rank] = expf(sv - m);
      if constexpr (MODE == kOutSample) sm.sz[rank] = sv + gumbel_from_word(nst.word(~(uint32_t)mine));
    }
  }
  __syncthreads();
  if (wid == 0) draw_or_cut<ROUTE, MODE>(a, r, sm, kk, pq, inv_t, m);
  if constexpr (MODE == kOutSample) return;
  __syncthreads();

  // ---- 5. log-probs: lp = x/T - m - ln Z_P on P (the first `cut` members of
  // K in the order: rank word at or above the last one's), -inf elsewhere
  const uint64_t lastw = sm.lastw;
  const float lzp = sm.lzp;
  if constexpr (MODE == kOutLogProbAt) {
    if (tid == 0) {
      const int64_t j = a.token_ids[r];
      float out = -__builtin_inff();
      if (j >= 0 && j < a.vocab) {
        const float x = static_cast<const float*>(a.logits)[src * a.row_stride + j];
        const uint32_t k = KeyF32::from_bits(__float_as_uint(x));
        if (k > KeyF32::kNegInf && rank_word(k, (int32_t)j) >= lastw) out = __fmul_rn(x, inv_t) - m - lzp;
      }
      a.out_lp[r] = out;
    }
  } else {
    f32x4* out_row = reinterpret_cast<f32x4*>(a.out_lp + (int64_t)r * a.vocab);
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const int vi = i * kB + tid;
      if (vi >= nvec) continue;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in_p = key[i][e] > KeyF32::kNegInf && rank_word(key[i][e], vi * 4 + e) >= lastw;
        o[e] = in_p ? __fmul_rn(d[i][e], inv_t) - m - lzp : -__builtin_inff();
      }
      out_row[vi] = f32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

}  // namespace

bool small_f32_supported(const RowArgs& a, DType dtype, Route route, OutMode mode) {
  // full log-prob rows go out as 16-byte stores
  const bool out_vec = mode != kOutLogProbFull || (reinterpret_cast<uintptr_t>(a.out_lp) % 16) == 0;
  return dtype == kF32 && (route == kRouteTopK || route == kRouteJoint) && out_vec &&
         a.vocab >= 4 && a.vocab <= (int64_t)kNV * 4 * kB && (a.vocab % 4) == 0 &&
         (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.logits) % 16) == 0;
}

namespace {
template <int ROUTE>
void launch_mode(const RowArgs& a, OutMode mode, hipStream_t stream) {
  const dim3 grid(a.n), block(kB);
  switch (mode) {
    case kOutSample:
      hipLaunchKernelGGL((rows_small_f32_kernel<ROUTE, kOutSample>), grid, block, 0, stream, a);
      break;
    case kOutLogProbFull:
      hipLaunchKernelGGL((rows_small_f32_kernel<ROUTE, kOutLogProbFull>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((rows_small_f32_kernel<ROUTE, kOutLogProbAt>), grid, block, 0, stream, a);
      break;
  }
}
}  // namespace

hipError_t launch_rows_small_f32(const RowArgs& a, Route route, OutMode mode, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  if (route == kRouteJoint)
    launch_mode<kRouteJoint>(a, mode, stream);
  else
    launch_mode<kRouteTopK>(a, mode, stream);
  return hipGetLastError();
}

}  // namespace tss
