// Host-side interface between the C ABI (tssample.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tss {

enum Route : int { kRouteNone = 0, kRouteTopK = 1, kRouteTopP = 2, kRouteJoint = 3 };
enum OutMode : int { kOutSample = 0, kOutLogProbFull = 1, kOutLogProbAt = 2 };
enum DType : int { kF32 = 0, kBF16 = 1 };

// Split-row kernels spread a row over at most kMaxSplit workgroups; each leaves
// one partial result in the handle's workspace.
constexpr int kMaxSplit = 64;
struct alignas(16) SplitPartial {
  uint32_t o;    // order word of the best entry (0: none)
  int32_t j;     // its index
  float s;       // its scaled logit
  float m;       // log-sum-exp of the part: max ...
  float sum;     // ... and sum of exp(s - max)
  uint32_t pad[3];
};

// Per-row state of the top-p route between its kernels.  Masses are relative
// to the reference m0 in base-2 units of the scaled logit s2 = x log2(e) / T:
// an entry weighs exp2(s2 - m0).
struct alignas(16) TopPRow {
  uint32_t mode;     // kTopPCut, kTopPAll (P = every entry above -inf) or kTopPDone
  int32_t bstar;     // histogram bucket holding the cutoff tie group (kTopPCut)
  float x_hi;        // entries with x >= x_hi lie above that bucket: members of P
  float x_lo;        // entries with x_lo <= x < x_hi lie in it
  float m0;          // mass reference
  float scale2;      // log2(e) / T
  float inv_w;       // buckets per base-2 unit
  float c;           // an entry's position in the histogram is fma(s2, -inv_w, c)
  float w;           // base-2 units per bucket, 1 / inv_w
  uint32_t nlist;    // entries of the cutoff bucket appended by the draw kernel
  int64_t src;       // source row in the logits buffer
  uint64_t seed;     // the request's seed
  uint64_t off;      // the request's Philox offset in this call
  double above;      // mass of the buckets above bstar (kTopPAll: of the whole row)
  double target;     // p times the row's mass
  double bscale;     // mass of one fixed-point unit of bucket bstar
  unsigned long long best;   // draw: max of (order of z2) << 32 | ~index over P's members
  // log-prob calls: P = {x >= x_cut} of mass zp (set by the finish kernel);
  // rows finished by the first kernel (kTopPDone) keep their greedy id in
  // done_id, or -1 for a row of NaN log-probs
  float x_cut;
  float inv_t;       // 1 / T
  int32_t done_id;
  double zp;
};
constexpr uint32_t kTopPCut = 0;
constexpr uint32_t kTopPDone = 1;
constexpr uint32_t kTopPAll = 2;

// One entry of a row's cutoff bucket.
struct alignas(8) TopPCand {
  uint32_t key;      // order key
  int32_t j;         // vocabulary index
};
constexpr int kTopPListCap = 256;   // cutoff-bucket entries kept per row

// Everything a row kernel needs; all pointers are device pointers.
struct RowArgs {
  const void* logits;
  int64_t row_stride;          // elements between rows
  int64_t vocab;
  int32_t n;                   // output rows
  const int32_t* gather;       // [n] or null
  const int32_t* req_map;      // [n] or null
  const float* temperature;    // [Q]
  const int32_t* top_k;        // [Q] (null on routes without top-k)
  const float* top_p;          // [Q] (null on routes without top-p)
  const uint64_t* seed;        // [Q]
  uint64_t step_offset;
  const uint64_t* req_offset;  // [Q] or null: per-request offsets added to step_offset
  int32_t* out_ids;            // sample: [n]
  float* out_lp;               // sample: [n] or null; log-probs: [n, vocab] or [n]
  const int32_t* token_ids;    // log-probs at ids: [n]
  int32_t mass_shift;          // fixed-point scale of probability masses: 2^mass_shift
  int32_t index_bits;          // ceil(log2(vocab)), at least 1
  uint32_t* split_counter;     // workspace: [max_rows] zeros between calls
  void* split_partials;        // workspace: [max_rows * kMaxSplit] SplitPartial
  TopPRow* topp_rows;          // workspace: [max_rows]
  TopPCand* topp_list;         // workspace: [max_rows * kTopPListCap]
  int32_t num_cu;              // compute units of the device (sizes persistent grids)
  int32_t heavy_first;         // fast kernel: workgroups take the rows without a register-
                               // resident top-k body first (more rows than CUs, n <= 1024)
};

// Philox offset of request q in this call.
__device__ __forceinline__ uint64_t noise_offset(const RowArgs& a, int64_t q) {
  return a.step_offset + (a.req_offset ? a.req_offset[q] : 0ull);
}

// Picks the kernel for a call (fast register-resident kernel where the row
// shape allows it, else the general multi-pass kernel) and launches it.
hipError_t launch_rows(const RowArgs& a, DType dtype, Route route, OutMode mode,
                       hipStream_t stream);

// Split-row kernel for calls whose every row is unfiltered (no-filter route).
bool split_none_supported(const RowArgs& a);
hipError_t launch_rows_split_none(const RowArgs& a, DType dtype, hipStream_t stream);
// Log-softmax of the raw rows at token_ids (same split kernel without noise);
// needs split_none_supported(a).
hipError_t launch_rows_raw_log_prob_at(const RowArgs& a, DType dtype, hipStream_t stream);

// Top-p route: a histogram kernel (one workgroup per row), a split draw kernel
// and a finishing kernel (one workgroup per row).
bool topp_supported(const RowArgs& a);
hipError_t launch_rows_topp(const RowArgs& a, DType dtype, hipStream_t stream);
// Log-probs (full rows or at ids) of rows filtered by top-p only or not at
// all, through the same cutoff: histogram, cutoff-bucket list, finish, and for
// full rows a write pass.
hipError_t launch_rows_topp_lp(const RowArgs& a, DType dtype, OutMode mode, hipStream_t stream);

// Short fp32 rows (up to 8192 entries) on the top-k and joint routes (sampling
// and log-probs): register-resident kernel, one workgroup per row.
bool small_f32_supported(const RowArgs& a, DType dtype, Route route, OutMode mode);
hipError_t launch_rows_small_f32(const RowArgs& a, Route route, OutMode mode, hipStream_t stream);

// The general multi-pass kernel alone (every row shape).
hipError_t launch_rows_general(const RowArgs& a, DType dtype, Route route, OutMode mode,
                               hipStream_t stream);

// Writes the speculative-verify request map (see ts_build_spec_map) to device memory.
hipError_t launch_spec_map(int32_t num_decode, int32_t num_prefill, int32_t num_spec,
                           int32_t* out_map, hipStream_t stream);

// Debug check of a call's device index arrays: clears *word, then ORs in
// kIndexGatherOut for a gather index outside [0, rows) and kIndexRequestOut
// for a request index outside [0, num_requests).
constexpr uint32_t kIndexGatherOut = 1u;
constexpr uint32_t kIndexRequestOut = 2u;
hipError_t launch_check_indices(int32_t n, const int32_t* gather, int64_t rows, const int32_t* req,
                                int32_t num_requests, uint32_t* word, hipStream_t stream);

// Chain verification of speculative drafts (one thread per request).
hipError_t launch_verify_chain(int32_t bs, int32_t n, const int32_t* candidates,
                               const int32_t* target_sampled, int32_t* predicts,
                               int32_t* accept_index, int32_t* accept_length, hipStream_t stream);

}  // namespace tss
