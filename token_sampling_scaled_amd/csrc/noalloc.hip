// ts_sample_noalloc: ts_sample without a handle, for callers that cannot
// allocate device memory.  The kernels' scratch memory (the split-row tickets,
// the partial results of split rows and the top-p route's per-row state) lives
// in one file-scope device array of fixed size; each GPU holds its own copy for
// the life of the process.  Host code never passes the array's name to a
// kernel: it takes the array's device address once per device with
// hipGetSymbolAddress and uses that address everywhere.
#include "tssample.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace {

constexpr int32_t kRows = TS_NOALLOC_MAX_ROWS;
constexpr size_t kCounterBytes = ((size_t)kRows * sizeof(uint32_t) + 255) & ~(size_t)255;
constexpr size_t kPartialBytes = (size_t)kRows * tss::kMaxSplit * sizeof(tss::SplitPartial);
constexpr size_t kTopPBytes = ((size_t)kRows * sizeof(tss::TopPRow) + 255) & ~(size_t)255;
constexpr size_t kListBytes = (size_t)kRows * tss::kTopPListCap * sizeof(tss::TopPCand);
constexpr size_t kScratchBytes = kCounterBytes + kPartialBytes + kTopPBytes + kListBytes;
static_assert(kPartialBytes % 256 == 0, "partials keep the 256-byte alignment");

// Tickets (zero between calls: the workgroup that merges a row puts its
// counter back), then the partial results, then the per-row top-p state and
// the top-p cutoff-bucket lists.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words(uint32_t* p, int32_t n) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  bool ready = false;
  unsigned char* ptr = nullptr;   // device address of this GPU's copy of `scratch`
  int32_t num_cu = 0;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

// Set-up on the current device, once: the array's device address, the CU
// count, and the tickets cleared by a fill kernel on the caller's stream (a
// kernel, not a memset, so that a first call under graph capture records a
// node that replays correctly).
ts_status device_scratch(hipStream_t stream, DeviceScratch* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TS_E_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ready) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return TS_E_HIP;
    }
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu < 1) {
      (void)hipGetLastError();
      return TS_E_HIP;
    }
    const int32_t words = (int32_t)(kCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return TS_E_HIP;
    d.ptr = static_cast<unsigned char*>(p);
    d.num_cu = cu;
    d.ready = true;
  }
  *out = d;
  return TS_OK;
}

int ceil_log2(int64_t v) {
  int b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}

}  // namespace

extern "C" ts_status ts_sample_noalloc(int64_t vocab, const void* logits, ts_dtype dtype,
                                       int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                                       const int32_t* gather_indices,
                                       const int32_t* token_to_request_index,
                                       const ts_params* params, uint64_t step_offset,
                                       int32_t no_top_k, int32_t no_top_p, int32_t* out_ids,
                                       float* out_logprob, void* stream) {
  if (vocab < 1 || vocab >= (int64_t(1) << 31) || params == nullptr) return TS_E_ARG;
  if (dtype != TS_F32 && dtype != TS_BF16) return TS_E_DTYPE;
  if (n < 0 || rows_in_buffer < 0) return TS_E_ARG;
  if (n > kRows) return TS_E_SIZE;
  if (row_stride < vocab) return TS_E_SIZE;
  if (gather_indices == nullptr && rows_in_buffer < n) return TS_E_SIZE;
  if (n == 0) return TS_OK;
  if (logits == nullptr || rows_in_buffer == 0 || out_ids == nullptr) return TS_E_ARG;
  if (params->temperature == nullptr || params->seed == nullptr || params->num_requests < 1)
    return TS_E_ARG;
  if (token_to_request_index == nullptr && params->num_requests < n) return TS_E_SIZE;
  if (!no_top_k && params->top_k == nullptr) return TS_E_ARG;
  if (!no_top_p && params->top_p == nullptr) return TS_E_ARG;

  const hipStream_t s = (hipStream_t)stream;
  DeviceScratch d;
  const ts_status st = device_scratch(s, &d);
  if (st != TS_OK) return st;

  tss::RowArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = vocab;
  a.n = n;
  a.gather = gather_indices;
  a.req_map = token_to_request_index;
  a.temperature = params->temperature;
  a.top_k = no_top_k ? nullptr : params->top_k;
  a.top_p = no_top_p ? nullptr : params->top_p;
  a.seed = params->seed;
  a.step_offset = step_offset;
  a.req_offset = params->step_offsets;
  a.out_ids = out_ids;
  a.out_lp = out_logprob;
  const int lb = ceil_log2(vocab);
  a.index_bits = lb < 1 ? 1 : lb;
  const int shift = 62 - ceil_log2(vocab + 1);
  a.mass_shift = shift > 44 ? 44 : shift;
  a.split_counter = reinterpret_cast<uint32_t*>(d.ptr);
  a.split_partials = d.ptr + kCounterBytes;
  a.topp_rows = reinterpret_cast<tss::TopPRow*>(d.ptr + kCounterBytes + kPartialBytes);
  a.topp_list = reinterpret_cast<tss::TopPCand*>(d.ptr + kCounterBytes + kPartialBytes + kTopPBytes);
  a.num_cu = d.num_cu;
  a.heavy_first = (n > d.num_cu && n <= 1024) ? 1 : 0;
  const tss::Route route = (tss::Route)ts_select_route(no_top_k, no_top_p);
  const hipError_t err =
      tss::launch_rows(a, dtype == TS_F32 ? tss::kF32 : tss::kBF16, route, tss::kOutSample, s);
  return err == hipSuccess ? TS_OK : TS_E_HIP;
}
