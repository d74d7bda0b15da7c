// Register-resident sampling kernel for bf16 rows (vocab <= 131072, vocab a
// multiple of 8, rows 16-byte aligned): one workgroup of 1024 threads (16
// waves) per output row; every logit is read from HBM exactly once with
// non-temporal 16-byte loads and kept in VGPRs.
//
// Rows with an active top-k (k <= 1024), with or without top-p.  The waves
// work independently while the row streams in -- data reaches the 16 waves of
// a workgroup at very different times, so no step waits for another wave until
// the row has arrived:
//   1. threshold: each wave issues the loads of the first half of its data,
//      then issues each load of the second half as a first-half vector
//      arrives (a wave blocked on a load issue could not work on data it
//      already holds), and takes t_w = the c-th largest of its 16-entry group
//      maxima over its first quarter (bitwise descent with ballots),
//      c = min(k, ceil(k/32) + 4);
//   2. filter: a 16-byte vector whose maximum reaches t_w is copied whole into
//      the wave's LDS segment (ballot + mbcnt), and its entries >= t_w are
//      counted in a histogram with one bin per bf16 value (a bin is exactly one
//      tie group);
//   3. after one barrier wave 0 scans the histogram from the top, down to
//      t* = max_w t_w (DPP prefix sums of counts and of the softmax mass
//      count * exp((x - x_max) / T)): the k-th value tau, the mass of K and the
//      top-p cutoff group.  Every entry >= t* was counted by its wave, so if
//      the count reaches k at or above t* then tau is the exact k-th largest
//      logit; otherwise the row takes the general body;
//   4. when the kept set ends inside the tie group at tau, the members of that
//      group are published and each one is ranked by index (one barrier);
//   5. the members of P are compacted over all waves (one atomic per wave);
//      Philox noise is drawn for P only -- by one wave when |P| <= 64, else one
//      member per thread -- and the perturbed argmax picks the id.
// Comparisons use the bf16 bit patterns as signed 16-bit integers: for positive
// values that is the value order and every negative value sorts below them, so
// it is exact whenever every t_w > +0.  A row with some t_w <= +0 runs steps
// 1-5 again on the row read again and taken to two's-complement order, with
// the patterns of |x| < 2^-64 sharing one histogram key (see sord2 and zkey);
// its wider, mostly empty window is scanned from per-block totals that every
// wave adds up (block_totals).  Rows without top-k run nok_row (the whole row
// in registers; top-p rows draw from a per-wave queue of member groups).
// Greedy rows
// take the first maximum.  Every other row -- k > 1024, NaN logits, a full LDS
// segment, fewer than k counted entries at or above t*, a cut inside the
// collapsed zone -- runs the general per-row body (general_row.hpp) on the
// same workgroup.
#include "general_row.hpp"

// Stage marks (a build with TSS_STAGE_MARKS defined only, a separate library):
// thread 0 of workgroup b < kStageRows (output row b, unless rows outnumber the
// compute units and heavy rows go first) records the device's constant-rate
// wall clock at each stage of the top-k body; the default build compiles the
// marks to nothing.
#ifdef TSS_STAGE_MARKS
namespace tss {
constexpr int kStageRows = 1024;
constexpr int kStageMarks = 16;
__device__ unsigned long long g_stage_marks[kStageRows * kStageMarks];
}  // namespace tss
#define TSS_MARK(k)                                                                       \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)::tss::kStageRows)                    \
      ::tss::g_stage_marks[blockIdx.x * ::tss::kStageMarks + (k)] = wall_clock64();       \
  } while (0)
// Copies the marks of workgroups [0, rows) to host memory ([rows][16] uint64:
// 0 start; top-k body: 1 threshold, 2 data offered, 3 counted, 4 scanned,
// 5 listed, 6 picked, 7 signed-order pass started; rows without top-k (sampling):
// 8 row maximum, 9 Z, 10 histogram counted, 11 cutoff found, 12 drawn (the
// race, for rows without top-p), 13 picked; 0 for a stage not reached since
// the last clear, else the last call's) and returns the wall clock's rate in
// kHz (0 on an error).
extern "C" int tss_stage_marks(unsigned long long* host, int rows) {
  if (host == nullptr || rows < 1 || rows > ::tss::kStageRows) return 0;
  if (hipDeviceSynchronize() != hipSuccess) return 0;
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(::tss::g_stage_marks),
                          sizeof(unsigned long long) * ::tss::kStageMarks * rows) != hipSuccess)
    return 0;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, 0) != hipSuccess) return 0;
  return khz;
}
// Clears the marks (between workloads).
extern "C" int tss_stage_marks_clear() {
  static const unsigned long long zeros[1024 * 16] = {};
  return hipMemcpyToSymbol(HIP_SYMBOL(::tss::g_stage_marks), zeros, sizeof(zeros)) == hipSuccess;
}
#else
#define TSS_MARK(k) \
  do {              \
  } while (0)
#endif

namespace tss {

namespace {

constexpr int kB = 1024;
constexpr int kWv = kB / kWave;
constexpr int kMaxK = 1024;
constexpr int kSegV = 256;                 // candidate vectors per wave
constexpr int kMaxTies = 1024;             // published members of the boundary tie group
constexpr int kHistBins = 32768;           // one bin per positive bf16 bit pattern
constexpr uint32_t kNegInfKey = 0x007Fu;
constexpr uint32_t kPosInfKey = 0xFF80u;
constexpr uint32_t kNegZeroKey = 0x7FFFu;
constexpr uint32_t kPosZeroKey = 0x8000u;
constexpr int32_t kPosInfBits = 0x7F80;    // bf16 +inf; larger positive patterns are NaN

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

struct FastShared {
  uint32_t hist[kHistBins / 2];    // 16-bit counters, two per word (at most 16 * kSegV * 8 counts)
  v4u cvec[kWv][kSegV];            // stored candidate vectors of each wave
  uint32_t cvim[kWv][kSegV];       // their vector index (i * 1024 + tid < 2^14, low half)
                                   // and maximum (bf16 bit pattern, high half)
  uint32_t pidx[kMaxK];            // kept set P: indices (each wave a range of its own)
  float pval[kMaxK];               //             logits
  uint32_t ties[kMaxTies];         // indices of the boundary tie group
  uint32_t wmax[kWv];              // per-wave maxima (same encoding)
  uint32_t wcount[kWv];
  float wz[kWv];
  float ws[kWv];
  int32_t wj[kWv];
  uint32_t flag;                   // nonzero: the row takes the general body
  uint32_t retry;                  // nonzero: a wave threshold <= +0 (raw patterns)
  int32_t tau_bits;                // scan results (wave 0)
  int32_t vc_bits;
  uint32_t need;
  uint32_t n_eq;
  float zp;
  uint32_t scan_ok;                // 0: general body, 1: go on, 2: signed-order pass
  uint32_t nties;
  uint32_t np;
  uint32_t tmax;                   // largest wave threshold published so far
  uint32_t kmax;                   // row maximum (unsigned image of the signed order)
  float mrow;                      // row maximum / T (scan result)
  uint32_t occ[4];                 // signed-order pass: bit b set when a counted key
                                   // lies in [256 b, 256 b + 255]
  uint32_t bcnt[128];              // signed-order pass, per occupied block of the window
  float bmass[128];                // (ordinal from the top): count and mass of its
                                   // entries in the window
};

// Rows without an active top-k: an exact histogram of order keys over the
// window [kmax - 32767, kmax] below the row maximum (one bin per bf16 value).
constexpr int kNoKBins = 32768;
constexpr int kNoKDrainEvery = 2;   // vectors between draws of the top-p draw's queue
// queued member groups per wave: fewer than 64 left over, plus 2 groups of
// every lane of kNoKDrainEvery vectors
constexpr int kNoKQueue = 64 + 2 * 64 * kNoKDrainEvery;
static_assert(3 * kNoKQueue * (1024 / 64) <= kNoKBins, "the queues live in the histogram's LDS");
struct NoKShared {
  uint32_t hist[kNoKBins];
  uint32_t wkey[kWv];
  uint32_t wnan[kWv];              // lanes of the wave holding a negative NaN
  float wz[kWv];
  float wpz[kWv];                  // per-wave race winners (no-filter rows)
  int32_t wpj[kWv];
  float wps[kWv];
  uint32_t vc_key;                 // the cutoff group's order key
  float zp;                        // mass of P in units of exp(x_max / T)
  uint32_t ok;                     // 0: the cutoff lies below the window
};

union RowShared {
  FastShared f;
  NoKShared n;
  general::Shared g;
};

// ---------------------------------------------------------------------------
// bf16 helpers

// Order keys of the two bf16 values packed in a dword (low half = lower index).
__device__ __forceinline__ uint32_t keys2(uint32_t u) {
  const uint32_t s = (u >> 15) & 0x00010001u;
  return u ^ ((s * 0xFFFFu) | 0x80008000u);
}

__device__ __forceinline__ uint32_t canon_key(uint32_t k) {
  return k == kNegZeroKey ? kPosZeroKey : k;
}

__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  const i16x2 x = __builtin_bit_cast(i16x2, a);
  const i16x2 y = __builtin_bit_cast(i16x2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Unsigned saturated a - b of both halves: a half is nonzero iff a > b there.
__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, a),
                                                                    __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ int32_t lo_i16(uint32_t u) { return (int32_t)(int16_t)(u & 0xFFFFu); }
__device__ __forceinline__ int32_t hi_i16(uint32_t u) { return ((int32_t)u) >> 16; }

// Largest of the eight bf16 bit patterns of a vector, as a signed 16-bit integer.
__device__ __forceinline__ int32_t vec_max_i16(const v4u& d) {
  const uint32_t m2 = pk_max_i16(pk_max_i16(d.x, d.y), pk_max_i16(d.z, d.w));
  return max(lo_i16(m2), hi_i16(m2));
}

__device__ __forceinline__ uint32_t word_of(const v4u& d, int w) {
  return w == 0 ? d.x : w == 1 ? d.y : w == 2 ? d.z : d.w;
}

__device__ __forceinline__ int32_t elem_i16(const v4u& d, int s) {
  const uint32_t w = word_of(d, s >> 1);
  return (s & 1) ? hi_i16(w) : lo_i16(w);
}

// Value of a bf16 bit pattern (sign-extended to 32 bits or not).
__device__ __forceinline__ float bits_value(int32_t b) { return __uint_as_float((uint32_t)b << 16); }

// Signed-order patterns: a bf16 pattern read as sign and magnitude, written as
// a two's-complement 16-bit integer (negative patterns become minus their 15
// magnitude bits, both zeros 0), so that comparing them as signed integers is
// the value order for every non-NaN value, with -0 and +0 equal (a positive
// NaN above +inf, a negative one below -inf).  sord2 maps the two patterns of
// a dword, sord16 one sign-extended pattern; sord_value16 takes one back to
// its raw pattern (+0 for both zeros).
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t sord2(uint32_t u) {
  const uint32_t neg = ((u >> 15) & 0x00010001u) * 0xFFFFu;   // 0xFFFF per negative half
  const u16x2 mag = __builtin_bit_cast(u16x2, u & 0x7FFF7FFFu);
  const uint32_t negm = __builtin_bit_cast(uint32_t, (u16x2){0, 0} - mag);   // per-half wrap
  return (u & ~neg) | (negm & neg);
}
__device__ __forceinline__ v4u sord4(const v4u& v) {
  return v4u{sord2(v.x), sord2(v.y), sord2(v.z), sord2(v.w)};
}
__device__ __forceinline__ int32_t sord16(int32_t b) { return b < 0 ? -(b & 0x7FFF) : b; }
__device__ __forceinline__ int32_t sord_value16(int32_t s) { return s < 0 ? ((-s) | 0x8000) : s; }
constexpr int32_t kNegInfOrd = -0x7F80;     // bf16 -inf in signed order

// Histogram keys of signed-order patterns: the patterns of |x| < 2^-64 (a
// biased exponent below 63, magnitude bits below kZone) share the key 0 and
// the others close up around it, so that 32768 consecutive keys span every
// pair of values of opposite signs that logits hold (say +1e4 down to
// -2^114).  zkey is monotone and one-to-one outside the zone; zkey_pat takes a
// key back to a pattern (0 for the zone), zkey_lo gives the smallest pattern
// with a key >= c.
constexpr int32_t kZone = 63 << 7;
__device__ __forceinline__ int32_t zkey(int32_t s) {
  return s >= kZone ? s - (kZone - 1) : (s <= -kZone ? s + (kZone - 1) : 0);
}
__device__ __forceinline__ int32_t zkey_pat(int32_t c) {
  return c > 0 ? c + (kZone - 1) : (c < 0 ? c - (kZone - 1) : 0);
}
__device__ __forceinline__ int32_t zkey_lo(int32_t c) {
  return c > 0 ? c + (kZone - 1) : c - (kZone - 1);
}
// Value of a pattern held raw (so false) or in signed order (so true).
__device__ __forceinline__ float pat_value(int32_t b, bool so) { return bits_value(so ? sord_value16(b) : b); }

// ---------------------------------------------------------------------------
// wave helpers

__device__ __forceinline__ uint32_t lane_rank(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// c-th largest (c >= 1) of the wave's values, 0 standing for "no value" (the
// result is 0 when fewer than c values exist).  Bitwise descent starting below
// the leading bits shared by the largest and smallest value.
template <int N>
__device__ __forceinline__ uint32_t wave_cth_largest16(const uint32_t (&vals)[N], uint32_t c) {
  uint32_t vmx = 0, vmn = 0xFFFFFFFFu, nnz = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    vmx = vals[i] > vmx ? vals[i] : vmx;
    vmn = (vals[i] != 0 && vals[i] < vmn) ? vals[i] : vmn;
    nnz += (uint32_t)__popcll(__ballot(vals[i] != 0));
  }
  if (nnz < c) return 0;
  vmx = wave_max_dpp(vmx);
  vmn = wave_min_dpp(vmn);
  const uint32_t diff = vmx ^ vmn;
  if (diff == 0) return vmx;
  const int top = 31 - __builtin_clz(diff);
  uint32_t prefix = vmx & ~((2u << top) - 1u);
  for (int b = top; b >= 0; --b) {
    const uint32_t trial = prefix | (1u << b);
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) cnt += (uint32_t)__popcll(__ballot(vals[i] >= trial));
    if (cnt >= c) prefix = trial;
  }
  return prefix;
}

struct Pick {
  float z;
  int32_t j;
  float s;
};


// Best (largest z, then smallest j) of the wave, returned in every lane.
__device__ __forceinline__ Pick wave_pick(Pick p) {
  const float zmax = wave_max_f32_dpp(p.z);
  const bool top = p.z == zmax;
  unsigned long long m = __ballot(top);
  if (__popcll(m) > 1) {   // equal scores: the smallest index among them
    const uint32_t jm = wave_min_dpp(top ? (uint32_t)p.j : 0xFFFFFFFFu);
    m = __ballot(top && (uint32_t)p.j == jm);
  }
  const int sl = __ffsll((long long)m) - 1;
  return Pick{zmax, __builtin_amdgcn_readlane(p.j, sl),
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.s), sl))};
}

// Block-wide best; the result is meaningful in wave 0 only.
__device__ __forceinline__ Pick block_pick(Pick p, FastShared& fs) {
  p = wave_pick(p);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    fs.wz[wid] = p.z;
    fs.wj[wid] = p.j;
    fs.ws[wid] = p.s;
  }
  __syncthreads();
  Pick b{-__builtin_inff(), 0x7FFFFFFF, 0.0f};
  if (wid == 0) {
    const int l = threadIdx.x & (kWave - 1);
    if (l < kWv) b = Pick{fs.wz[l], fs.wj[l], fs.ws[l]};
    b = wave_pick(b);
  }
  return b;
}

__device__ __forceinline__ void write_result(const RowArgs& a, int r, int32_t id, float lp) {
  a.out_ids[r] = id;
  if (a.out_lp) a.out_lp[r] = lp;
}

// Greedy row: first index of the largest logit.
template <int NV>
__device__ __forceinline__ void greedy_row(const RowArgs& a, int r, int nvec, const v4u (&d)[NV],
                                           FastShared& fs) {
  uint32_t best = 0;
  int32_t bj = 0x7FFFFFFF;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int32_t e0 = (i * kB + (int)threadIdx.x) * 8;
    if (e0 >= nvec * 8) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t k2 = keys2(word_of(d[i], w));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t k = canon_key(h ? (k2 >> 16) : (k2 & 0xFFFFu));
        if (k > kPosInfKey) k = 0;   // NaN reads as -inf
        const int32_t j = e0 + 2 * w + h;
        if (k > best || (k == best && j < bj)) {
          best = k;
          bj = j;
        }
      }
    }
  }
  const Pick p = block_pick(Pick{(float)best, bj, 0.0f}, fs);   // keys < 2^16 are exact in fp32
  if (threadIdx.x == 0) {
    if (p.z <= (float)kNegInfKey)
      write_result(a, r, -1, __builtin_nanf(""));
    else
      write_result(a, r, p.j, 0.0f);
  }
}

// ---------------------------------------------------------------------------
// histogram of positive bf16 bit patterns, 16-bit counters packed two per word

__device__ __forceinline__ void hist_add(uint32_t* hist, int32_t bits) {
  atomicAdd(&hist[bits >> 1], 1u << ((bits & 1) * 16));
}

__device__ __forceinline__ uint32_t hist_get(const uint32_t* hist, int32_t bits) {
  return (hist[bits >> 1] >> ((bits & 1) * 16)) & 0xFFFFu;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Result of the histogram scan (identical in every wave).
struct ScanOut {
  bool ok;            // false: fewer than k counted entries in [lo, hi]
  int32_t tau_bits;   // the k-th value
  uint32_t need;      // members of its tie group inside K (lowest indices)
  uint32_t n_eq;      // size of that tie group
  int32_t vc_bits;    // the top-p cutoff value (P = K and x >= cutoff)
  float zp;           // mass of P in units of exp(x_max / T)
};

// Softmax weight exp(x / T - m) of the entries of bin b: the raw pattern b
// (so false), or the key b - hoff of signed-order patterns (so true; the
// entries of the zone of |x| < 2^-64 weigh as x = 0, a relative change of
// their weight below 2^-64 / T).
__device__ __forceinline__ float bin_weight(int32_t b, float inv_t, float m, int32_t hoff, bool so) {
  return __expf(__fmaf_rn(bits_value(so ? sord_value16(zkey_pat(b - hoff)) : b), inv_t, -m));
}

// Whether any of the bins [max(top - 255, lo), top] may hold an entry, from
// the occupancy bits of the 256-key blocks (occ_lo: blocks 0..63, occ_hi:
// 64..127; wave-uniform).  The chunk meets at most two blocks.
__device__ __forceinline__ bool chunk_occupied(uint64_t occ_lo, uint64_t occ_hi, int32_t top,
                                               int32_t lo) {
  const int32_t bh = top >> 8;
  const int32_t bl = (top - 255 > lo ? top - 255 : lo) >> 8;
  const uint64_t mh = bh < 64 ? occ_lo >> bh : occ_hi >> (bh - 64);
  const uint64_t ml = bl < 64 ? occ_lo >> bl : occ_hi >> (bl - 64);
  return ((mh | ml) & 1u) != 0;
}

// The highest occupied block below block i (i <= 128), or -1.
__device__ __forceinline__ int32_t occupied_below(uint64_t occ_lo, uint64_t occ_hi, int32_t i) {
  if (i > 64) {
    const uint64_t mh = i >= 128 ? occ_hi : occ_hi & ((1ull << (i - 64)) - 1ull);
    if (mh) return 127 - (int32_t)__clzll((long long)mh);
  }
  const uint64_t ml = i >= 64 ? occ_lo : occ_lo & ((1ull << i) - 1ull);
  return ml ? 63 - (int32_t)__clzll((long long)ml) : -1;
}

// Next chunk top after an empty chunk ending at top (bins >= lo): the top of
// the highest occupied block below it, plus 256 for the loop's step; below
// lo when no occupied block remains.
__device__ __forceinline__ int32_t skip_empty(uint64_t occ_lo, uint64_t occ_hi, int32_t top,
                                              int32_t lo) {
  const int32_t nb = occupied_below(occ_lo, occ_hi, (top - 255 > lo ? top - 255 : lo) >> 8);
  return nb < 0 ? lo - 1 + 4 * kWave : nb * 256 + 255 + 4 * kWave;
}

// Counts and masses of the occupied 256-key blocks of the window [lo, hi]
// (hi the top bin of a block), the block of ordinal o (from the top) taken by
// wave o mod 16, as the scan below adds them up; every wave returns the
// number of such blocks.  The one-wave scan then starts at the blocks where k
// and the top-p mass are reached instead of walking every block above them.
__device__ __forceinline__ int32_t block_totals(const uint32_t* hist, const uint32_t* occ,
                                                uint32_t* bcnt, float* bmass, int32_t lo,
                                                int32_t hi, float inv_t, float m, int32_t hoff,
                                                int wid, int lane) {
  const uint64_t occ_lo = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[0]) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[1]) << 32);
  const uint64_t occ_hi = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[2]) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[3]) << 32);
  int32_t ord = 0;
  for (int32_t b = occupied_below(occ_lo, occ_hi, (hi >> 8) + 1); b >= (lo >> 8);
       b = occupied_below(occ_lo, occ_hi, b), ++ord) {
    if ((ord & (kWv - 1)) != wid) continue;
    const int32_t top = b * 256 + 255;
    uint32_t cs = 0;
    float ms = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t bin = top - (4 * lane + i);
      const uint32_t c = bin >= lo ? hist_get(hist, bin) : 0u;
      const float w = bin_weight(bin, inv_t, m, hoff, true);
      cs += c;
      ms += c ? (float)c * w : 0.0f;
    }
    const uint32_t ci = wave_scan_u32(cs);
    const float mi = wave_scan_f32(ms);
    if (lane == kWave - 1) {
      bcnt[ord] = ci;
      bmass[ord] = mi;
    }
  }
  return ord;
}

// Scan the bins [lo, hi] (hi = the row maximum's) from the top; with so (wide
// windows of signed-order keys, mostly empty), the scan jumps from an empty
// chunk to the highest occupied 256-key block (occ) below it.
// Lane l takes bins top - 4l .. top - 4l - 3 of each 256-bin chunk.  When the
// k-th value falls in the first chunk (the common case) the top-p cutoff is
// found from the same registers; otherwise a second pass recomputes the masses.
// The cutoff group is the first one, from the top, whose cumulative K-mass
// reaches p * Z_K; the top group is always kept.
// With a block index (nblk >= 0: block_totals' counts and masses, hi a
// block's top), the first pass starts at the block where the count reaches k
// and the second at the block where the mass reaches p * Z_K.
__device__ __forceinline__ ScanOut scan_hist(const uint32_t* hist, const uint32_t* occ,
                                             int32_t lo, int32_t hi, float inv_t, float m,
                                             uint32_t k, bool p_on, float p, int32_t hoff,
                                             bool so, const uint32_t* bcnt = nullptr,
                                             const float* bmass = nullptr, int32_t nblk = -1) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t occ_lo = 0, occ_hi = 0;
  if (so) {
    occ_lo = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[0]) |
             ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[1]) << 32);
    occ_hi = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[2]) |
             ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)occ[3]) << 32);
  }
  ScanOut o{false, 0, 0, 0, 0, 0.0f};
  uint32_t cbase = 0, n_gt = 0;
  float mbase = 0.0f, mass_gt = 0.0f;
  bool in_first = true;
  int32_t top1 = hi;
  // block index: lane l holds blocks l and 64 + l (inclusive prefixes)
  const bool bidx = so && nblk >= 0;
  float f0 = 0.0f, f1 = 0.0f;
  int32_t ok_blk = 0;
  if (bidx) {
    const uint32_t c0 = lane < nblk ? bcnt[lane] : 0u;
    const uint32_t c1 = lane + kWave < nblk ? bcnt[lane + kWave] : 0u;
    const float m0 = lane < nblk ? bmass[lane] : 0.0f;
    const float m1 = lane + kWave < nblk ? bmass[lane + kWave] : 0.0f;
    const uint32_t i0 = wave_scan_u32(c0);
    const uint32_t i1 = wave_scan_u32(c1) + (uint32_t)__builtin_amdgcn_readlane((int)i0, kWave - 1);
    f0 = wave_scan_f32(m0);
    f1 = wave_scan_f32(m1) + readlane_f(f0, kWave - 1);
    const unsigned long long h0 = __ballot(i0 >= k), h1 = __ballot(i1 >= k);
    if (!h0 && !h1) return o;   // fewer than k entries in the window
    ok_blk = h0 ? __ffsll((long long)h0) - 1 : kWave + __ffsll((long long)h1) - 1;
    const uint32_t inc = ok_blk < kWave ? (uint32_t)__builtin_amdgcn_readlane((int)i0, ok_blk)
                                        : (uint32_t)__builtin_amdgcn_readlane((int)i1, ok_blk - kWave);
    const uint32_t own = ok_blk < kWave ? (uint32_t)__builtin_amdgcn_readlane((int)c0, ok_blk)
                                        : (uint32_t)__builtin_amdgcn_readlane((int)c1, ok_blk - kWave);
    cbase = inc - own;
    const int32_t pb = ok_blk - 1;
    mbase = pb < 0 ? 0.0f : pb < kWave ? readlane_f(f0, pb) : readlane_f(f1, pb - kWave);
    // the ok_blk-th occupied block from the top
    int32_t b = occupied_below(occ_lo, occ_hi, (hi >> 8) + 1);
    for (int32_t t = 0; t < ok_blk; ++t) b = occupied_below(occ_lo, occ_hi, b);
    top1 = b * 256 + 255;
    in_first = top1 == hi;
  }
  uint32_t cc[4];
  float mm[4], mx[4];   // per bin: count, mass, mass of the bins above it
  for (int32_t top = top1; top >= lo; top -= 4 * kWave) {
    if (so && !chunk_occupied(occ_lo, occ_hi, top, lo)) {   // an empty chunk: nothing to add up
      in_first = false;
      top = skip_empty(occ_lo, occ_hi, top, lo);
      continue;
    }
    uint32_t cs = 0;
    float ms = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t b = top - (4 * lane + i);
      const uint32_t h = hist_get(hist, b > 0 ? b : 0);   // unconditional: the reads overlap
      cc[i] = b >= lo ? h : 0u;
      const float w = bin_weight(b, inv_t, m, hoff, so);
      mm[i] = cc[i] ? (float)cc[i] * w : 0.0f;
      cs += cc[i];
      ms += mm[i];
    }
    const uint32_t ci = wave_scan_u32(cs);
    const float mi = wave_scan_f32(ms);
    uint32_t cex = cbase + ci - cs;
    float mex = mbase + (mi - ms);
    int32_t hit = -1;
    uint32_t h_gt = 0, h_eq = 0;
    float h_mgt = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = mex;
      if (cex < k && cex + cc[i] >= k) {   // at most one bin of the row crosses k
        hit = top - (4 * lane + i);
        h_gt = cex;
        h_eq = cc[i];
        h_mgt = mex;
      }
      cex += cc[i];
      mex += mm[i];
    }
    const unsigned long long hm = __ballot(hit >= 0);
    if (hm) {
      const int sl = __ffsll((long long)hm) - 1;
      o.ok = true;
      o.tau_bits = __builtin_amdgcn_readlane(hit, sl);
      n_gt = (uint32_t)__builtin_amdgcn_readlane((int)h_gt, sl);
      o.n_eq = (uint32_t)__builtin_amdgcn_readlane((int)h_eq, sl);
      mass_gt = readlane_f(h_mgt, sl);
      break;
    }
    cbase += (uint32_t)__builtin_amdgcn_readlane((int)ci, kWave - 1);
    mbase += readlane_f(mi, kWave - 1);
    in_first = false;
  }
  if (!o.ok) return o;
  o.need = k - n_gt;
  const float zk = mass_gt + (float)o.need * bin_weight(o.tau_bits, inv_t, m, hoff, so);
  o.vc_bits = o.tau_bits;
  o.zp = zk;
  if (!p_on) return o;
  const float target = p * zk;
  if (in_first) {
    int32_t hit = -1;
    float h_z = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t b = hi - (4 * lane + i);
      const float cum = (b == o.tau_bits) ? zk : mx[i] + mm[i];
      if (hit < 0 && b >= o.tau_bits && cc[i] != 0 && cum >= target &&
          (mx[i] < target || b == hi)) {
        hit = b;
        h_z = cum;
      }
    }
    const unsigned long long hm = __ballot(hit >= 0);
    if (hm) {
      const int sl = __ffsll((long long)hm) - 1;
      o.vc_bits = __builtin_amdgcn_readlane(hit, sl);
      o.zp = readlane_f(h_z, sl);
    }
    return o;
  }
  float mb = 0.0f;
  int32_t top2 = hi;
  if (bidx) {
    // the first block from the top whose cumulative mass reaches the target
    // (with a margin for the order of the additions), at the latest the k-th
    // value's block
    const float tm = target * (1.0f - 0x1p-10f);
    const unsigned long long g0 = __ballot(lane < ok_blk && f0 >= tm);
    const unsigned long long g1 = __ballot(lane + kWave < ok_blk && f1 >= tm);
    const int32_t pb = g0 ? __ffsll((long long)g0) - 1 : g1 ? kWave + __ffsll((long long)g1) - 1 : ok_blk;
    mb = pb == 0 ? 0.0f : pb - 1 < kWave ? readlane_f(f0, pb - 1) : readlane_f(f1, pb - 1 - kWave);
    int32_t b = occupied_below(occ_lo, occ_hi, (hi >> 8) + 1);
    for (int32_t t = 0; t < pb; ++t) b = occupied_below(occ_lo, occ_hi, b);
    top2 = b * 256 + 255;
  }
  for (int32_t top = top2; top >= o.tau_bits; top -= 4 * kWave) {
    // an empty chunk (the bin at tau is never empty): nothing to add up
    if (so && !chunk_occupied(occ_lo, occ_hi, top, o.tau_bits)) {
      top = skip_empty(occ_lo, occ_hi, top, o.tau_bits);
      continue;
    }
    bool ne[4];
    float ms = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t b = top - (4 * lane + i);
      const uint32_t h = hist_get(hist, b > 0 ? b : 0);
      const uint32_t cnt = b > o.tau_bits ? h : 0u;
      ne[i] = cnt != 0 || b == o.tau_bits;
      const float w = bin_weight(b, inv_t, m, hoff, so);
      mm[i] = cnt ? (float)cnt * w : 0.0f;
      ms += mm[i];
    }
    const float mi = wave_scan_f32(ms);
    float mex = mb + (mi - ms);
    int32_t hit = -1;
    float h_z = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t b = top - (4 * lane + i);
      const float cum = (b == o.tau_bits) ? zk : mex + mm[i];
      if (hit < 0 && b >= o.tau_bits && ne[i] && cum >= target && (mex < target || b == hi)) {
        hit = b;
        h_z = cum;
      }
      mex += mm[i];
    }
    const unsigned long long hm = __ballot(hit >= 0);
    if (hm) {
      const int sl = __ffsll((long long)hm) - 1;
      o.vc_bits = __builtin_amdgcn_readlane(hit, sl);
      o.zp = readlane_f(h_z, sl);
      break;
    }
    mb += readlane_f(mi, kWave - 1);
  }
  return o;
}

// The wave's lanes read LDS entries other lanes of the same wave have just
// written.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of published tie-group indices below j.
__device__ __forceinline__ uint32_t tie_rank(const uint32_t* ties, uint32_t nt, uint32_t j) {
  uint32_t rank = 0;
  const v4u* t4 = reinterpret_cast<const v4u*>(ties);
  for (uint32_t t = 0; t < nt; t += 4) {
    const v4u v = t4[t >> 2];
    rank += (v.x < j ? 1u : 0u) + ((t + 1 < nt && v.y < j) ? 1u : 0u) +
            ((t + 2 < nt && v.z < j) ? 1u : 0u) + ((t + 3 < nt && v.w < j) ? 1u : 0u);
  }
  return rank;
}

// Order key (16 bits) back to the bf16 value it stands for.
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t bits = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
  return __uint_as_float(bits << 16);
}

// A row without an active top-k, whole row in registers (d).  P is every
// finite entry, or with top-p the tie groups from the top whose mass before
// them stays below p * Z.  Then, by MODE: the perturbed argmax over P (sample),
// every entry's log-prob of the processed distribution written from the
// registers (full rows: one read and one write of the row), or the log-prob
// at the request's token id.  Returns false when the row needs the general
// body instead (NaN or +inf in the row, or a top-p cutoff below the window of
// 32768 order keys under the row maximum); the caller then synchronises first.
// Every pass works on the raw order keys of two entries at a time (packed
// 16-bit maxima, minima and saturated differences); -0 and +0, whose keys
// differ by one, are told apart only where an entry is counted or drawn.
template <int NV, int MODE>
__device__ __forceinline__ bool nok_row(const RowArgs& a, int r, int nvec, int nfull, const v4u (&d)[NV],
                        float inv_t, bool p_on, float pq, uint64_t seed, uint64_t off,
                        RowShared& sh) {
  NoKShared& ns_ = sh.n;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  // ---- largest and smallest order key (positive NaN sorts above +inf,
  // negative NaN below -inf)
  uint32_t kmx2 = 0u, kmn2 = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (!(i < nfull || i * kB + tid < nvec)) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t k2 = keys2(word_of(d[i], w));
      kmx2 = pk_max_u16(kmx2, k2);
      kmn2 = pk_min_u16(kmn2, k2);
    }
  }
  uint32_t kmx = canon_key(max(kmx2 & 0xFFFFu, kmx2 >> 16));
  const uint32_t kmn = min(kmn2 & 0xFFFFu, kmn2 >> 16);
  kmx = wave_max_dpp(kmx);
  const uint32_t nan_lo = (uint32_t)__popcll(__ballot(kmn < kNegInfKey));
  if (lane == 0) {
    ns_.wkey[wid] = kmx;
    ns_.wnan[wid] = nan_lo;
  }
  if (p_on) {                        // clear the histogram meanwhile
    v4u* h4 = reinterpret_cast<v4u*>(ns_.hist);
#pragma unroll
    for (int i = 0; i < kNoKBins / 4 / kB; ++i) h4[i * kB + tid] = v4u{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  kmx = wave_max_dpp(lane < kWv ? ns_.wkey[lane] : 0u);
  TSS_MARK(8);
  const uint32_t any_nan_lo = wave_max_dpp(lane < kWv ? ns_.wnan[lane] : 0u);
  if (kmx >= kPosInfKey || any_nan_lo != 0) return false;   // NaN or +inf: general body
  if (kmx <= kNegInfKey) {                        // no finite entry: id -1 and lp NaN
    if (MODE == kOutSample) {
      if (tid == 0) write_result(a, r, -1, __builtin_nanf(""));
    } else if (MODE == kOutLogProbAt) {
      if (tid == 0) a.out_lp[r] = __builtin_nanf("");
    } else {                                      // a NaN row of log-probs
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      f32x4* out_row = reinterpret_cast<f32x4*>(a.out_lp + (int64_t)r * a.vocab);
      const float qn = __builtin_nanf("");
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = i * kB + tid;
        if (!(i < nfull || vi < nvec)) continue;
        out_row[2 * vi] = f32x4{qn, qn, qn, qn};
        out_row[2 * vi + 1] = f32x4{qn, qn, qn, qn};
      }
    }
    return true;
  }
  // base-2 units: s2 = x log2(e) / T; exp2(s2 - m2) = exp(x / T - m)
  const float sc2 = 1.4426950408889634f * inv_t;
  const float m2 = key_value(kmx) * sc2;
  const float m = __fmul_rn(key_value(kmx), inv_t);

  if (MODE == kOutSample && !p_on) {
    // ---- P = every finite entry: Z and the perturbed argmax in one pass.
    // argmax_j (x_j / T + g_j), g_j = -ln(-ln u_j), is the winner of an
    // exponential race: argmin_j E_j / w_j with w_j = exp2(s2_j - m2) (the
    // terms of Z) and E_j = -log2 u_j (-ln u_j times log2 e, one factor for
    // every j).  j beats the best b so far when E_j w_b < E_b w_j: no
    // division, and one logarithm per entry besides the exp2 Z needs anyway.
    // -inf entries weigh 0 and never win.  Z adds the same terms in the same
    // order as the two-pass form below.
    const NoiseStream nst{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r,
                          (uint32_t)off, (uint32_t)(off >> 32)};
    float z = 0.0f, eb = 1.0f, wb = 0.0f, xb = 0.0f;
    int32_t jb = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * kB + tid;
      if (!(i < nfull || vi < nvec)) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Philox4 wds = nst.block((uint32_t)(2 * vi + h));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = word_of(d[i], 2 * h + (e >> 1));
          const float x = __uint_as_float((e & 1) ? (u & 0xFFFF0000u) : (u << 16));
          const float w = __builtin_amdgcn_exp2f(__fmaf_rn(x, sc2, -m2));
          z += w;
          const float ee = -__builtin_amdgcn_logf(uniform_from_word(wds.v[e]));
          if (ee * wb < eb * w) {          // j rises within a thread: ties keep the first
            eb = ee;
            wb = w;
            xb = x;
            jb = vi * 8 + 4 * h + e;
          }
        }
      }
    }
    // the thread's winner as a base-2 score log2 w - log2 E (w > 0: the row
    // holds a finite entry, which weighs at least as much as exp2(0) = 1 at
    // its maximum, so some thread's wb is positive; a thread with none keeps -inf)
    Pick p{wb > 0.0f ? __builtin_amdgcn_logf(wb) - __builtin_amdgcn_logf(eb) : -__builtin_inff(), jb,
           __fmul_rn(xb, inv_t)};
    TSS_MARK(12);
    z = wave_sum(z);
    p = wave_pick(p);
    if (lane == 0) {
      ns_.wz[wid] = z;
      ns_.wpz[wid] = p.z;
      ns_.wpj[wid] = p.j;
      ns_.wps[wid] = p.s;
    }
    __syncthreads();
    if (wid == 0) {
      float zt = 0.0f;
#pragma unroll
      for (int w = 0; w < kWv; ++w) zt += ns_.wz[w];
      Pick b{-__builtin_inff(), 0x7FFFFFFF, 0.0f};
      if (lane < kWv) b = Pick{ns_.wpz[lane], ns_.wpj[lane], ns_.wps[lane]};
      b = wave_pick(b);
      if (lane == 0) write_result(a, r, b.j, b.s - m - __logf(zt));
      TSS_MARK(13);
    }
    return true;
  }

  // ---- Z = sum over finite entries of exp(x / T - m) (exp2 of -inf is 0)
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (!(i < nfull || i * kB + tid < nvec)) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t u = word_of(d[i], w);
      z += __builtin_amdgcn_exp2f(__fmaf_rn(__uint_as_float(u << 16), sc2, -m2));
      z += __builtin_amdgcn_exp2f(__fmaf_rn(__uint_as_float(u & 0xFFFF0000u), sc2, -m2));
    }
  }
  z = wave_sum(z);
  if (lane == 0) ns_.wz[wid] = z;
  __syncthreads();
  TSS_MARK(9);
  z = 0.0f;
#pragma unroll
  for (int w = 0; w < kWv; ++w) z += ns_.wz[w];

  uint32_t vc_key = kNegInfKey + 1;               // P: every finite entry
  float zp = z;
  if (p_on) {
    // ---- exact histogram of the entries in the window that can be in P:
    // the entries with s < m + ln((1 - p) Z / V) weigh less than (1 - p) Z
    // together, so the cutoff is never below them.  The smallest order key
    // whose value passes that test (a binary search: the test is monotone in
    // the key, and -0 passes exactly when +0 does) bounds the counted keys.
    const uint32_t wlo = kmx > (uint32_t)(kNoKBins - 1) ? kmx - (uint32_t)(kNoKBins - 1) : 1u;
    const float s_lo = m + __logf(fmaxf(1.0f - pq, 0.0f) * z / (float)a.vocab);
    uint32_t klo = max(wlo, kNegInfKey + 1), khi = kmx;   // kmx itself always passes
    while (klo < khi) {
      const uint32_t mid = (klo + khi) >> 1;
      if (__fmul_rn(key_value(mid), inv_t) >= s_lo) khi = mid;
      else klo = mid + 1;
    }
    const uint32_t kthr = klo;
    const i16x2 below2 = __builtin_bit_cast(i16x2, (kthr - 1u) * 0x10001u);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (!(i < nfull || i * kB + tid < nvec)) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t k2 = keys2(word_of(d[i], w));
        // halves >= kthr leave a nonzero unsigned saturated difference
        const uint32_t hit = pk_sub_sat_u16(k2, __builtin_bit_cast(uint32_t, below2));
        if (hit) {
          if (hit & 0xFFFFu) atomicAdd(&ns_.hist[canon_key(k2 & 0xFFFFu) - wlo], 1u);
          if (hit >> 16) atomicAdd(&ns_.hist[canon_key(k2 >> 16) - wlo], 1u);
        }
      }
    }
    __syncthreads();
    TSS_MARK(10);
    // ---- wave 0 scans the bins from the maximum down: the cutoff group is
    // the first nonempty one whose cumulative mass reaches p Z (the top group
    // is always kept)
    if (wid == 0) {
      const float target = pq * z;
      float mbase = 0.0f;
      uint32_t hit_key = 0;
      float hit_z = 0.0f;
      bool found = false;
      for (int32_t top = (int32_t)kmx; top >= (int32_t)wlo && !found; top -= 4 * kWave) {
        float mm[4];
        uint32_t cc[4];
        float ms = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t b = top - (4 * lane + i);
          cc[i] = b >= (int32_t)wlo ? ns_.hist[b - (int32_t)wlo] : 0u;
          mm[i] = cc[i] ? (float)cc[i] * __builtin_amdgcn_exp2f(__fmaf_rn(key_value((uint32_t)b), sc2, -m2))
                        : 0.0f;
          ms += mm[i];
        }
        const float mi = wave_scan_f32(ms);
        float mex = mbase + (mi - ms);
        int32_t hit = -1;
        float h_z = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t b = top - (4 * lane + i);
          const float cum = mex + mm[i];
          if (hit < 0 && cc[i] != 0 && cum >= target && (mex < target || b == (int32_t)kmx)) {
            hit = b;
            h_z = cum;
          }
          mex += mm[i];
        }
        const unsigned long long hm = __ballot(hit >= 0);
        if (hm) {
          const int sl = __ffsll((long long)hm) - 1;
          hit_key = (uint32_t)__builtin_amdgcn_readlane(hit, sl);
          hit_z = readlane_f(h_z, sl);
          found = true;
        }
        mbase += readlane_f(mi, kWave - 1);
      }
      if (lane == 0) {
        ns_.ok = found ? 1u : 0u;
        ns_.vc_key = hit_key;
        ns_.zp = hit_z;
      }
    }
    __syncthreads();
    if (ns_.ok == 0) return false;
    TSS_MARK(11);
    vc_key = ns_.vc_key;
    zp = ns_.zp;
  }

  // the members of P: canonical key >= vc_key, that is raw key >= raw_thr
  // (-0 too when the cutoff group is +0's)
  const uint32_t raw_thr = vc_key == kPosZeroKey ? kNegZeroKey : vc_key;
  if (MODE != kOutSample) {
    // lp = x / T - m - ln Z_P on P, -inf elsewhere
    const float lzp = __logf(zp);
    auto lp_of_key = [&](uint32_t k) -> float {
      return k >= raw_thr ? __fmul_rn(key_value(k), inv_t) - m - lzp : -__builtin_inff();
    };
    if (MODE == kOutLogProbAt) {
      if (tid == 0) {
        const int64_t j = a.token_ids[r];
        float out = -__builtin_inff();
        if (j >= 0 && j < a.vocab) {
          const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
          const uint16_t rb = reinterpret_cast<const uint16_t*>(a.logits)[src * a.row_stride + j];
          out = lp_of_key(keys2((uint32_t)rb) & 0xFFFFu);
        }
        a.out_lp[r] = out;
      }
      return true;
    }
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4* out_row = reinterpret_cast<f32x4*>(a.out_lp + (int64_t)r * a.vocab);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * kB + tid;
      if (!(i < nfull || vi < nvec)) continue;
      float o[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t k2 = keys2(word_of(d[i], w));
        o[2 * w] = lp_of_key(k2 & 0xFFFFu);
        o[2 * w + 1] = lp_of_key(k2 >> 16);
      }
      // plain stores (the L2 merges the two halves of every line)
      out_row[2 * vi] = f32x4{o[0], o[1], o[2], o[3]};
      out_row[2 * vi + 1] = f32x4{o[4], o[5], o[6], o[7]};
    }
    return true;
  }

  // ---- Philox noise for the members of P (x at or above the cutoff group's
  // value: -0 with +0, never -inf), perturbed argmax.  Each wave queues its
  // 4-entry groups holding a member, with their raw words, in LDS (the
  // histogram's, free by now) from a ballot, and draws one Philox block per
  // queued group, 64 at a time: every lane of a draw holds a member group,
  // where drawing in place ran the block for every lane whenever one of them
  // held a member.
  const float x_thr = key_value(vc_key);
  const NoiseStream nst{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r,
                        (uint32_t)off, (uint32_t)(off >> 32)};
  uint32_t* qg = ns_.hist + wid * (3 * kNoKQueue);   // queued group ids
  uint32_t* qw = qg + kNoKQueue;                     // their two raw words each
  float bz = -__builtin_inff(), bs = 0.0f;
  int32_t bj = 0x7FFFFFFF;
  uint32_t fill = 0;                                  // queued groups (wave-uniform)
  auto drain_from = [&](uint32_t first, uint32_t count) {   // draw count (<= 64) queued groups
    if ((uint32_t)lane < count) {
      const uint32_t q = first + (uint32_t)lane;
      const uint32_t g = qg[q];
      const uint32_t ua = qw[2 * q], ub = qw[2 * q + 1];
      const float x[4] = {__uint_as_float(ua << 16), __uint_as_float(ua & 0xFFFF0000u),
                          __uint_as_float(ub << 16), __uint_as_float(ub & 0xFFFF0000u)};
      const Philox4 wds = nst.block(g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!(x[e] >= x_thr)) continue;
        const float sv = __fmul_rn(x[e], inv_t);
        const float zz = sv + gumbel_from_word(wds.v[e]);
        const int32_t j = (int32_t)(g * 4u + (uint32_t)e);
        if (better(zz, j, bz, bj)) {
          bz = zz;
          bj = j;
          bs = sv;
        }
      }
    }
  };
  // every kNoKDrainEvery vectors: draw the full rounds of 64 queued groups and
  // move the rest to the front
  auto drain_rounds = [&]() {
    wave_lds_sync();
    uint32_t first = 0;
    for (; fill - first >= (uint32_t)kWave; first += kWave) drain_from(first, kWave);
    const uint32_t rest = fill - first;
    uint32_t mg = 0, ma = 0, mb2 = 0;
    if ((uint32_t)lane < rest) {
      mg = qg[first + lane];
      ma = qw[2 * (first + lane)];
      mb2 = qw[2 * (first + lane) + 1];
    }
    __builtin_amdgcn_wave_barrier();
    if ((uint32_t)lane < rest) {
      qg[lane] = mg;
      qw[2 * lane] = ma;
      qw[2 * lane + 1] = mb2;
    }
    fill = rest;
  };
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = i * kB + tid;
    const bool valid = i < nfull || vi < nvec;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // entries 4h .. 4h + 3 of the vector: one Philox block
      const uint32_t ua = word_of(d[i], 2 * h), ub = word_of(d[i], 2 * h + 1);
      const float xm = fmaxf(fmaxf(__uint_as_float(ua << 16), __uint_as_float(ua & 0xFFFF0000u)),
                             fmaxf(__uint_as_float(ub << 16), __uint_as_float(ub & 0xFFFF0000u)));
      const bool mem = valid && xm >= x_thr;
      const unsigned long long mm = __ballot(mem);
      if (mem) {
        const uint32_t pos = fill + lane_rank(mm);
        qg[pos] = (uint32_t)(2 * vi + h);
        qw[2 * pos] = ua;
        qw[2 * pos + 1] = ub;
      }
      fill += (uint32_t)__popcll(mm);
    }
    if ((i + 1) % kNoKDrainEvery == 0 && i + 1 < NV) drain_rounds();
  }
  wave_lds_sync();
  for (uint32_t first = 0; first < fill; first += kWave)
    drain_from(first, fill - first < (uint32_t)kWave ? fill - first : (uint32_t)kWave);
  TSS_MARK(12);
  Pick best{bz, bj, bs};
  best = block_pick(best, sh.f);
  if (tid == 0) write_result(a, r, best.j, best.s - m - __logf(zp));
  TSS_MARK(13);
  return true;
}

// The row of this workgroup when a call has more rows than the device has
// CUs: one workgroup of this kernel fills a CU, so the rows of the workgroups
// dispatched last start only when earlier ones end.  Rows that take the
// register-resident top-k body (or greedy sampling) end within a few
// microseconds of their data; the others (no top-k: Philox noise for the
// whole row or its nucleus; k > 1024, greedy log-probs: the general body) can
// take several times as long.  So workgroup b takes the b-th heavy row (in
// row order), and after the heavy rows the light ones: a permutation of the
// rows that changes no result, only the order rows start in.  Needs n <= 1024
// (one row per thread of the classification).
template <int ROUTE, int MODE>
__device__ __forceinline__ int heavy_first_row(const RowArgs& a, uint64_t* cls) {
  constexpr bool kHasK = (ROUTE == kRouteTopK || ROUTE == kRouteJoint);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  bool heavy = false;
  if (tid < a.n) {
    const int64_t qt = a.req_map ? (int64_t)a.req_map[tid] : (int64_t)tid;
    const float t = a.temperature[qt];
    const int32_t k = kHasK ? a.top_k[qt] : 0;
    const bool greedy = !(t >= 1e-5f);
    const bool light = greedy ? MODE == kOutSample
                              : (kHasK && k >= 1 && (int64_t)k < a.vocab && k <= kMaxK);
    heavy = !light;
  }
  const uint64_t bm = __ballot(heavy);
  if (lane == 0) cls[wid] = bm;
  __syncthreads();
  uint32_t nh = 0;
#pragma unroll
  for (int w = 0; w < kWv; ++w) nh += (uint32_t)__popcll(cls[w]);
  const uint32_t b = blockIdx.x;
  const bool want_heavy = b < nh;
  uint32_t idx = want_heavy ? b : b - nh;       // rank of the row within its class
  int r = -1;
#pragma unroll
  for (int w = 0; w < kWv; ++w) {
    const int left = a.n - w * kWave;           // rows of this wave's slice
    const uint64_t valid = left >= kWave ? ~0ull : (left <= 0 ? 0ull : ((1ull << left) - 1ull));
    const uint64_t m = want_heavy ? cls[w] : (~cls[w] & valid);
    const uint32_t c = (uint32_t)__popcll(m);
    if (r < 0) {
      if (idx < c) {
        const unsigned long long hit = __ballot(((m >> lane) & 1ull) && lane_rank(m) == idx);
        r = w * kWave + (__ffsll((long long)hit) - 1);
      } else {
        idx -= c;
      }
    }
  }
  return r >= 0 ? r : (int)blockIdx.x;   // always found: b < n and the classes split [0, n)
}

// Whether a row with a wave threshold at or below +0 takes the signed-order
// second pass (else the general body): every instance but full-row log-probs
// on the joint route at 16 vectors a thread, where a second copy of the steps
// beside the register-resident row makes the first copy spill.
template <int NV, int ROUTE, int MODE>
constexpr bool kSignedPass = !(MODE == kOutLogProbFull && ROUTE == kRouteJoint && NV == 16);

// Outcome of the top-k steps: the row is done, the steps run again in signed
// order, or the general body takes the row (after a barrier, once every wave
// is done with the fast path's shared memory).
constexpr int kBodyDone = 0, kBodyRetry = 1, kBodyGeneral = 2;

// Steps 1-6 of a row with an active top-k (k <= kMaxK), the first NB vectors
// of the row in d (the steps issue the other loads).  Comparisons use the bf16
// patterns as signed 16-bit integers: raw patterns (sgn false) are in value
// order only above +0, so in sampling mode a row with a wave threshold <= +0
// returns true and the caller runs the steps again with sgn true, on the row
// read again and taken to signed order (sord2) as each vector arrives.  The
// histogram's bin of a signed-order pattern s is then zkey(s) + hoff, over the
// 32768 keys below the row maximum's; a cut (the k-th value or the top-p
// cutoff) in the zone of |x| < 2^-64 sends the row to the general body.  Both
// passes stream the row the same way, so that neither needs more registers.
template <int NV, int ROUTE, int MODE, bool sgn>
__device__ __forceinline__ int topk_body(const RowArgs& a, int r, int64_t src, int64_t q,
                                          const v4u* row, int nvec, int nfull, v4u (&d)[NV],
                                          int32_t kq, float pq, bool p_on, uint64_t seed,
                                          float inv_t, RowShared& sh) {
  // the wave threshold comes from the first NQ vectors (a quarter of the row
  // when NV >= 4), in groups of GV vectors (16 entries)
  constexpr int NB = NV >= 2 ? NV / 2 : 1;
  constexpr int NQ = NV >= 4 ? NV / 4 : NB;
  constexpr int GV = NQ >= 2 ? 2 : 1;
  constexpr int NG = NQ / GV;
  constexpr uint32_t kDiv = 8u * NV / NQ;   // c ~ 2k * (share of the row in the sample)
  FastShared& fs = sh.f;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  // clear the histogram while the loads are in flight
  {
    v4u* h4 = reinterpret_cast<v4u*>(fs.hist);
#pragma unroll
    for (int i = 0; i < kHistBins / 8 / kB; ++i) h4[i * kB + tid] = v4u{0u, 0u, 0u, 0u};
    if (tid == 0) {
      fs.flag = 0;
      fs.retry = 0;
      fs.nties = 0;
      fs.np = 0;
      fs.tmax = 0;
      fs.kmax = 0;
    }
    if constexpr (sgn) {
      if (tid < 4) fs.occ[tid] = 0;
    }
  }
  __syncthreads();

  // ---- 1. this wave's threshold, from the first NQ vectors of its data
  int32_t vmax = -32768;           // running maximum bit pattern (signed 16-bit order)
  int32_t vm[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if constexpr (sgn) d[i] = sord4(d[i]);
    vm[i] = (i < nfull || tid < nvec - i * kB) ? vec_max_i16(d[i]) : -32768;
    vmax = max(vmax, vm[i]);
    if (NB + i < NV) {
      __builtin_amdgcn_sched_barrier(0);
      const int vi = (NB + i) * kB + tid;
      d[NB + i] = __builtin_nontemporal_load(row + (vi < nvec ? vi : nvec - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  uint32_t gm[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int32_t mg = vm[g * GV];
#pragma unroll
    for (int v = 1; v < GV; ++v) mg = max(mg, vm[g * GV + v]);
    gm[g] = (uint32_t)(mg + 0x8000);           // unsigned image of the signed order
  }
  const uint32_t cq = ((uint32_t)kq + kDiv - 1) / kDiv + 4;
  const uint32_t c = (uint32_t)kq < cq ? (uint32_t)kq : cq;
  const uint32_t tw = wave_cth_largest16<NG>(gm, c);
  // raw patterns: the signed order is the value order only above +0.  Signed
  // order: the threshold must lie above -inf (so that no -inf or NaN entry can
  // be counted).
  const int32_t t16w = (int32_t)tw - 0x8000;
  const bool wave_ok = tw != 0 && (sgn ? t16w > kNegInfOrd : t16w > 0);
  // t* = max_w t_w is where the scan stops, so an entry below the largest
  // threshold published so far can never matter: filter with that one
  uint32_t teff = tw;
  if (lane == 0) {
    if (!wave_ok) {
      if (!sgn && tw != 0 && kSignedPass<NV, ROUTE, MODE>) fs.retry = 1;
      else fs.flag = 1;
    }
    if (wave_ok) teff = max(tw, atomicMax(&fs.tmax, tw));
  }
  teff = (uint32_t)__builtin_amdgcn_readfirstlane((int)teff);
  const int32_t t16 = (int32_t)teff - 0x8000;

  // ---- 2. filter vectors into this wave's segment as they arrive, then count
  // their entries
  TSS_MARK(1);                      // threshold
  uint32_t wfill = 0;               // wave-uniform number of vectors offered
  v4u* my_vec = fs.cvec[wid];
  uint32_t* my_vim = fs.cvim[wid];
  auto offer = [&](int i, int32_t mv) {
    const bool cand = mv >= t16;
    const unsigned long long bm = __ballot(cand);
    if (bm) {
      const uint32_t pos = wfill + lane_rank(bm);
      if (cand && pos < (uint32_t)kSegV) {
        my_vec[pos] = d[i];
        my_vim[pos] = (uint32_t)(i * kB + tid) | ((uint32_t)mv << 16);
      }
      wfill += (uint32_t)__popcll(bm);
    }
  };
  // a wave without a usable threshold sends the row to the general body:
  // nothing of it is stored or counted
  if (wave_ok) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) offer(i, vm[i]);
#pragma unroll
    for (int i = NQ; i < NV; ++i) {
      if constexpr (sgn) d[i] = sord4(d[i]);
      const int32_t mv = (i < nfull || tid < nvec - i * kB) ? vec_max_i16(d[i]) : -32768;
      vmax = max(vmax, mv);
      if (i < NB && NB + i < NV) {
        __builtin_amdgcn_sched_barrier(0);
        const int vi = (NB + i) * kB + tid;
        d[NB + i] = __builtin_nontemporal_load(row + (vi < nvec ? vi : nvec - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
      offer(i, mv);
    }
  }
  TSS_MARK(2);                      // the wave's data all in and offered
  if (lane == 0 && wfill > (uint32_t)kSegV) fs.flag = 1;   // a full segment lost vectors
  const uint32_t stored = wfill < (uint32_t)kSegV ? wfill : (uint32_t)kSegV;
  // signed order: the row maximum places the histogram's window before any
  // entry is counted, and nothing below the window is
  int32_t hoff = 0, tlo = -32768;
  if constexpr (sgn) {
    const uint32_t wmaxu = wave_max_dpp((uint32_t)(vmax + 0x8000));
    if (lane == 0) atomicMax(&fs.kmax, wmaxu);
    __syncthreads();
    hoff = 0x7FFF - zkey((int32_t)fs.kmax - 0x8000);
    tlo = zkey_lo(-hoff);
  }
  {
    // entries >= the largest threshold published by now (<= t*) go into the
    // histogram; stored vectors whose maximum is below it are skipped
    wave_lds_sync();
    const int32_t tc = max(max(t16, (int32_t)fs.tmax - 0x8000), tlo);
    const i16x2 tc2 = __builtin_bit_cast(i16x2, (uint32_t)tc * 0x10001u);
    // signed order: also mark the key's 256-key block, so that the scan passes
    // over the empty stretches of the wide window without reading them
    auto count_key = [&](int32_t key) {
      hist_add(fs.hist, key);
      if constexpr (sgn) atomicOr(&fs.occ[key >> 13], 1u << ((key >> 8) & 31));
    };
    for (uint32_t e = lane; e < stored; e += kWave) {
      const int32_t vmx = (int32_t)my_vim[e] >> 16;
      if (vmx < tc) continue;
      const v4u dv = my_vec[e];
      // entries below tc: sign bits of the saturated packed differences
      uint32_t nlt = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        nlt += (uint32_t)__popc(__builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(
                                    __builtin_bit_cast(i16x2, word_of(dv, w)), tc2)) & 0x80008000u);
      if (nlt == 7) {                // the maximum is the only entry >= tc
        count_key(sgn ? zkey(vmx) + hoff : vmx);
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int32_t val = elem_i16(dv, s);
          if (val >= tc) count_key(sgn ? zkey(val) + hoff : val);
        }
      }
    }
  }
  const uint32_t wmaxu = wave_max_dpp((uint32_t)(vmax + 0x8000));
  if (lane == 0) {
    fs.wcount[wid] = stored;
    fs.wmax[wid] = wmaxu;
    atomicMax(&fs.kmax, wmaxu);
  }
  __syncthreads();
  TSS_MARK(3);                      // counted, first barrier

  // ---- 3. wave 0 scans the histogram from the row maximum down to t* = max_w t_w
  // (signed order: after every wave has added up some of the window's
  // occupied blocks)
  int32_t nblk = -1;
  if constexpr (sgn) {
    const int32_t kmax16 = (int32_t)fs.kmax - 0x8000;
    const int32_t tstar16 = (int32_t)fs.tmax - 0x8000;
    const int32_t lo = max(zkey(tstar16), -hoff) + hoff;
    const int32_t hi = zkey(kmax16) + hoff;
    if (fs.flag == 0 && kmax16 <= kPosInfBits && (hi & 255) == 255 && lo <= hi)
      nblk = block_totals(fs.hist, fs.occ, fs.bcnt, fs.bmass, lo, hi, inv_t,
                          __fmul_rn(pat_value(kmax16, true), inv_t), hoff, wid, lane);
    __syncthreads();
  }
  float m = 0.0f;                   // row maximum / T (wave 0)
  if (wid == 0) {
    // the row maximum and t* = max_w t_w, published with LDS atomics (a wave
    // without a usable threshold set the flag, so t* is the maximum of all)
    const uint32_t kmaxu = fs.kmax;
    const uint32_t tstaru = fs.tmax;
    const int32_t kmax16 = (int32_t)kmaxu - 0x8000;
    const int32_t tstar16 = (int32_t)tstaru - 0x8000;
    m = __fmul_rn(pat_value(kmax16, sgn), inv_t);
    // a wave threshold <= +0 (raw patterns, sampling): signed-order pass
    const bool retry = kSignedPass<NV, ROUTE, MODE> && !sgn && fs.retry != 0;
    const bool usable = !retry && fs.flag == 0 && kmax16 <= kPosInfBits;   // no NaN, no full segment
    ScanOut so{false, 0, 0, 0, 0, 0.0f};
    if (usable) {
      const int32_t lo = sgn ? max(zkey(tstar16), -hoff) + hoff : tstar16;
      const int32_t hi = sgn ? zkey(kmax16) + hoff : kmax16;
      so = scan_hist(fs.hist, fs.occ, lo, hi, inv_t, m, (uint32_t)kq, p_on, pq, hoff, sgn, fs.bcnt,
                     fs.bmass, nblk);
      if constexpr (sgn) {
        // keys back to patterns; a cut in the zone has no exact pattern
        if (so.tau_bits == hoff || so.vc_bits == hoff) so.ok = false;
        so.tau_bits = zkey_pat(so.tau_bits - hoff);
        so.vc_bits = zkey_pat(so.vc_bits - hoff);
      }
    }
    if (lane == 0) {
      fs.scan_ok = retry ? 2u : so.ok ? 1u : 0u;
      fs.tau_bits = so.tau_bits;
      fs.vc_bits = so.vc_bits;
      fs.need = so.need;
      fs.n_eq = so.n_eq;
      fs.zp = so.zp;
      fs.mrow = m;
    }
  }
  __syncthreads();
  TSS_MARK(4);                      // scanned, second barrier
  const uint32_t scan_ok = fs.scan_ok;
  if (scan_ok != 1u)
    return (kSignedPass<NV, ROUTE, MODE> && !sgn && scan_ok == 2u) ? kBodyRetry : kBodyGeneral;
  const int32_t tau = fs.tau_bits;
  const int32_t vc = fs.vc_bits;
  const uint32_t need = fs.need;

  if constexpr (MODE != kOutSample) {
    // ---- log-probs of the processed distribution: lp = x/T - m - ln Z_P on
    // P, -inf elsewhere, written from the registers (full rows), or at one id
    const bool tie_cut = vc == tau && need < fs.n_eq;
    uint32_t nt = 0;
    if (tie_cut) {
      // publish the tie group at tau: its `need` lowest indices are in P
      const uint32_t stored_t = (int32_t)fs.wmax[wid] - 0x8000 >= tau ? stored : 0u;
      for (uint32_t e = lane; e < stored_t; e += kWave) {
        const uint32_t vim = my_vim[e];
        if (((int32_t)vim >> 16) < tau) continue;
        const v4u dv = my_vec[e];
        const uint32_t vi = vim & 0xFFFFu;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          if (elem_i16(dv, sl) == tau) {
            const uint32_t slot = atomicAdd(&fs.nties, 1u);
            if (slot < (uint32_t)kMaxTies) fs.ties[slot] = vi * 8 + (uint32_t)sl;
          }
        }
      }
      __syncthreads();
      nt = fs.nties;
      if (nt > (uint32_t)kMaxTies) {
        return kBodyGeneral;
      }
    }
    const float mrow = fs.mrow;
    const float lzp = __logf(fs.zp);
    const int32_t thr = tie_cut ? tau + 1 : vc;
    auto lp_of = [&](int32_t val, uint32_t j) -> float {
      bool keep = val >= thr;
      if (tie_cut && val == tau) keep = tie_rank(fs.ties, nt, j) < need;
      return keep ? __fmul_rn(pat_value(val, sgn), inv_t) - mrow - lzp : -__builtin_inff();
    };
    if (MODE == kOutLogProbAt) {
      if (tid == 0) {
        const int64_t j = a.token_ids[r];
        float out = -__builtin_inff();
        if (j >= 0 && j < a.vocab) {
          const uint16_t raw = reinterpret_cast<const uint16_t*>(a.logits)[src * a.row_stride + j];
          const int32_t pat = (int32_t)(int16_t)raw;
          out = lp_of(sgn ? sord16(pat) : pat, (uint32_t)j);
        }
        a.out_lp[r] = out;
      }
      return kBodyDone;
    }
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4* out_row = reinterpret_cast<f32x4*>(a.out_lp + (int64_t)r * a.vocab);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * kB + tid;
      if (!(i < nfull || vi < nvec)) continue;
      float o[8];
      // the second pass reads its row a third time here rather than keep it
      // in registers through the steps (a second register-resident copy of
      // them does not fit without spills)
      v4u dv = d[i];
      if constexpr (sgn) dv = sord4(__builtin_nontemporal_load(row + vi));
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) o[sl] = lp_of(elem_i16(dv, sl), (uint32_t)(vi * 8 + sl));
      // plain stores: each of the two lands at a 32-byte stride, and the L2
      // merges both halves of every line before it goes to HBM (non-temporal
      // stores leave half-filled lines: 68 us instead of 39 us per call at
      // 256 x 128256)
      out_row[2 * vi] = f32x4{o[0], o[1], o[2], o[3]};
      out_row[2 * vi + 1] = f32x4{o[4], o[5], o[6], o[7]};
    }
    return kBodyDone;
  }
  const uint64_t off = noise_offset(a, q);
  const NoiseStream ns{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r,
                       (uint32_t)off, (uint32_t)(off >> 32)};

  // ---- 4. each wave lists its stored vectors whose maximum reaches vc (they
  // hold the members of P) with one atomic; when P ends inside the tie group
  // at tau, that group's indices are published as well
  const bool tie_cut = vc == tau && need < fs.n_eq;
  uint32_t* mvlist = fs.pidx;                          // listed slots (w * kSegV + e)
  constexpr int kChunks = (kSegV + kWave - 1) / kWave;
  const uint32_t stored_mine = (int32_t)fs.wmax[wid] - 0x8000 >= vc ? stored : 0u;
  {
    bool listed[kChunks];
    uint32_t tot = 0;
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      const uint32_t e = (uint32_t)(ch * kWave + lane);
      listed[ch] = false;
      if ((uint32_t)(ch * kWave) < stored_mine) {      // wave-uniform
        const uint32_t vim = e < stored_mine ? my_vim[e] : 0x80000000u;
        listed[ch] = ((int32_t)vim >> 16) >= vc;
        if (listed[ch] && tie_cut) {
          const v4u dv = my_vec[e];
          const uint32_t vi = vim & 0xFFFFu;
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) {
            if (elem_i16(dv, sl) == tau) {
              const uint32_t slot = atomicAdd(&fs.nties, 1u);
              if (slot < (uint32_t)kMaxTies) fs.ties[slot] = vi * 8 + (uint32_t)sl;
            }
          }
        }
        tot += (uint32_t)__popcll(__ballot(listed[ch]));
      }
    }
    if (tot) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&fs.np, tot);
      base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        if ((uint32_t)(ch * kWave) >= stored_mine) break;
        const unsigned long long bm = __ballot(listed[ch]);
        const uint32_t pos = base + lane_rank(bm);
        if (listed[ch] && pos < (uint32_t)kMaxK)
          mvlist[pos] = (uint32_t)(wid * kSegV + ch * kWave + lane);
        base += (uint32_t)__popcll(bm);
      }
    }
  }
  __syncthreads();
  TSS_MARK(5);                      // listed, third barrier
  const uint32_t nmv = fs.np;
  const uint32_t nt = tie_cut ? fs.nties : 0u;
  if (nmv > (uint32_t)kMaxK || nt > (uint32_t)kMaxTies) {
    return kBodyGeneral;
  }

  // ---- 5. one listed vector per thread: its members (x >= thr outright; of
  // the tie group at tau, when P ends inside it, the `need` lowest indices)
  // draw their noise.  At most 64 listed vectors: wave 0 alone, else every
  // wave and a block argmax.
  const bool one_wave = nmv <= (uint32_t)kWave;
  if (one_wave && wid != 0) return kBodyDone;
  const int32_t thr = tie_cut ? tau + 1 : vc;
  const int32_t eqv = tie_cut ? tau : 0x7FFFFFFF;
  Pick best{-__builtin_inff(), 0x7FFFFFFF, 0.0f};
  if ((uint32_t)tid < nmv) {
    const uint32_t f = mvlist[tid];
    const uint32_t w = f / kSegV;
    const uint32_t e = f - w * kSegV;
    const v4u dv = fs.cvec[w][e];
    const uint32_t vi = fs.cvim[w][e] & 0xFFFFu;
    uint32_t mk = 0, eq = 0;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int32_t val = elem_i16(dv, sl);
      mk |= (val >= thr ? 1u : 0u) << sl;
      eq |= (val == eqv ? 1u : 0u) << sl;
    }
    while (eq) {
      const int sl = __ffs(eq) - 1;
      eq &= eq - 1;
      if (tie_rank(fs.ties, nt, vi * 8 + (uint32_t)sl) < need) mk |= 1u << sl;
    }
    while (mk) {
      const int sl = __ffs(mk) - 1;
      mk &= mk - 1;
      const uint32_t j = vi * 8 + (uint32_t)sl;
      const float sv = __fmul_rn(pat_value(elem_i16(dv, sl), sgn), inv_t);
      const float z = sv + gumbel_from_word(ns.word(j));
      if (z > best.z || (z == best.z && (int32_t)j < best.j)) best = Pick{z, (int32_t)j, sv};
    }
  }
  if (one_wave) {
    best = wave_pick(best);
    if (lane == 0) write_result(a, r, best.j, best.s - m - __logf(fs.zp));
    TSS_MARK(6);                    // drawn and picked
    return kBodyDone;
  }
  best = block_pick(best, fs);
  if (tid == 0) write_result(a, r, best.j, best.s - m - __logf(fs.zp));
  TSS_MARK(6);                      // drawn and picked
  return kBodyDone;
}

template <int NV, int ROUTE, int MODE>
__global__ __launch_bounds__(kB) void rows_fast_bf16_kernel(RowArgs a) {
  constexpr bool kHasK = (ROUTE == kRouteTopK || ROUTE == kRouteJoint);
  constexpr bool kHasP = (ROUTE == kRouteTopP || ROUTE == kRouteJoint);
  // loads in flight: the first NB vectors, then (in the steps) one more per
  // arriving vector
  constexpr int NB = NV >= 2 ? NV / 2 : 1;
  __shared__ RowShared sh;
  __shared__ uint64_t cls[kWv];
  FastShared& fs = sh.f;

  TSS_MARK(0);                      // start
  const int r = a.heavy_first ? heavy_first_row<ROUTE, MODE>(a, cls) : (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
  const int64_t q = a.req_map ? (int64_t)a.req_map[r] : (int64_t)r;
  const v4u* row = reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(a.logits) +
                                                src * a.row_stride);
  const int nvec = (int)(a.vocab >> 3);
  const int nfull = nvec / kB;       // vector slots every thread of the row holds

  // ---- stream the row into registers.  Slots past the row re-read its last
  // vector and are ignored where used, so every load is unconditional and
  // each vector is waited for on its own at its first use.  The first half is
  // issued before the request's parameters are even read (they decide the
  // body, and waiting for them first would delay every load by one memory
  // latency); the second half goes out one load per arriving first-half vector.
  v4u d[NV];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int vi = i * kB + tid;
    d[i] = __builtin_nontemporal_load(row + (vi < nvec ? vi : nvec - 1));
  }

  const float temp = a.temperature[q];
  const int32_t kq = kHasK ? a.top_k[q] : 0;
  const float pq = kHasP ? a.top_p[q] : 1.0f;
  const uint64_t seed = a.seed[q];   // read up front: a late load would stall the tail
  const bool greedy = !(temp >= 1e-5f);
  const bool k_on = kHasK && kq >= 1 && (int64_t)kq < a.vocab;
  const bool p_on = kHasP && pq < 1.0f - 1e-6f;

  // Rows without top-k: register-resident, below (noise for P, or the
  // log-probs written from the registers).  k above kMaxK, and greedy rows
  // asked for log-probs: general body.
  const bool nok = !greedy && !k_on;
  int st = kBodyGeneral;             // uniform over the workgroup
  if ((!greedy && !nok && (!k_on || kq > kMaxK)) || (greedy && MODE != kOutSample)) {
    // general body from the start
  } else if (greedy || nok) {
#pragma unroll
    for (int i = NB; i < NV; ++i) {
      const int vi = i * kB + tid;
      d[i] = __builtin_nontemporal_load(row + (vi < nvec ? vi : nvec - 1));
    }
    if (greedy) {
      greedy_row<NV>(a, r, nvec, d, fs);
      st = kBodyDone;
    } else {
      st = nok_row<NV, MODE>(a, r, nvec, nfull, d, 1.0f / temp, p_on, pq, seed, noise_offset(a, q), sh)
               ? kBodyDone : kBodyGeneral;
    }
  } else {
    const float inv_t = 1.0f / temp;
    st = topk_body<NV, ROUTE, MODE, false>(a, r, src, q, row, nvec, nfull, d, kq, pq, p_on, seed,
                                           inv_t, sh);
    if (kSignedPass<NV, ROUTE, MODE> && st == kBodyRetry) {
      // a wave threshold <= +0: the steps again, in signed order, on the row read again
      TSS_MARK(7);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int vi = i * kB + tid;
        d[i] = __builtin_nontemporal_load(row + (vi < nvec ? vi : nvec - 1));
      }
      st = topk_body<NV, ROUTE, MODE, true>(a, r, src, q, row, nvec, nfull, d, kq, pq, p_on, seed,
                                            inv_t, sh);
    }
  }
  if (st == kBodyGeneral) {
    __syncthreads();
    general::general_row<uint16_t, ROUTE, MODE>(a, r, sh.g);
  }
}

template <int NV>
hipError_t launch_nv(const RowArgs& a, Route route, OutMode mode, hipStream_t stream) {
  const dim3 grid(a.n), block(kB);
  if (mode == kOutLogProbFull) {
    switch (route) {
      case kRouteNone:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteNone, kOutLogProbFull>), grid, block, 0, stream, a);
        break;
      case kRouteTopK:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteTopK, kOutLogProbFull>), grid, block, 0, stream, a);
        break;
      case kRouteTopP:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteTopP, kOutLogProbFull>), grid, block, 0, stream, a);
        break;
      default:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteJoint, kOutLogProbFull>), grid, block, 0, stream, a);
        break;
    }
    return hipGetLastError();
  }
  if (mode == kOutLogProbAt) {
    switch (route) {
      case kRouteNone:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteNone, kOutLogProbAt>), grid, block, 0, stream, a);
        break;
      case kRouteTopK:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteTopK, kOutLogProbAt>), grid, block, 0, stream, a);
        break;
      case kRouteTopP:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteTopP, kOutLogProbAt>), grid, block, 0, stream, a);
        break;
      default:
        hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteJoint, kOutLogProbAt>), grid, block, 0, stream, a);
        break;
    }
    return hipGetLastError();
  }
  switch (route) {
    case kRouteNone:
      hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteNone, kOutSample>), grid, block, 0, stream, a);
      break;
    case kRouteTopK:
      hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteTopK, kOutSample>), grid, block, 0, stream, a);
      break;
    case kRouteTopP:
      hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteTopP, kOutSample>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((rows_fast_bf16_kernel<NV, kRouteJoint, kOutSample>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rows(const RowArgs& a, DType dtype, Route route, OutMode mode,
                       hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  // every row unfiltered: noise for every entry, rows split over workgroups
  if (mode == kOutSample && route == kRouteNone && split_none_supported(a))
    return launch_rows_split_none(a, dtype, stream);
  // every row top-p filtered (or unfiltered): cutoff per row, then a split draw
  if (mode == kOutSample && route == kRouteTopP && topp_supported(a))
    return launch_rows_topp(a, dtype, stream);
  const bool aligned = (reinterpret_cast<uintptr_t>(a.logits) % 16) == 0 && (a.row_stride % 8) == 0;
  const int64_t nvec = a.vocab / 8;
  // full log-prob rows go out as 16-byte stores
  const bool out_vec = mode != kOutLogProbFull || (reinterpret_cast<uintptr_t>(a.out_lp) % 16) == 0;
  const bool fast_shape = dtype == kBF16 && aligned && (a.vocab % 8) == 0 && nvec <= 16 * (int64_t)kB &&
                          out_vec;
  // log-probs of rows without top-k in any other shape (fp32 above all): the
  // top-p route's cutoff, then a write pass
  if (mode != kOutSample && (route == kRouteTopP || route == kRouteNone) && !fast_shape &&
      topp_supported(a))
    return launch_rows_topp_lp(a, dtype, mode, stream);
  // the fast kernel: sampling on every route but top-p only; log-probs on
  // every route (rows without an active top-k write them from registers)
  const bool fast_route = mode == kOutSample ? route != kRouteTopP : true;
  if (fast_shape && fast_route) {
    const int64_t per = (nvec + kB - 1) / kB;
    if (per <= 1) return launch_nv<1>(a, route, mode, stream);
    if (per <= 2) return launch_nv<2>(a, route, mode, stream);
    if (per <= 4) return launch_nv<4>(a, route, mode, stream);
    if (per <= 8) return launch_nv<8>(a, route, mode, stream);
    return launch_nv<16>(a, route, mode, stream);
  }
  // short fp32 rows with top-k: their own register-resident kernel
  if (small_f32_supported(a, dtype, route, mode)) return launch_rows_small_f32(a, route, mode, stream);
  return launch_rows_general(a, dtype, route, mode, stream);
}

}  // namespace tss
