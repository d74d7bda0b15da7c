// C ABI of the sampler: argument checks, filter-route choice from the host
// flags, and the launch on the caller's stream.  See include/tssample.h for the
// contract of every entry point.
#include "tssample.h"

#include <hip/hip_runtime.h>

#include <new>

#include "launch.hpp"

struct ts_sampler {
  int64_t vocab;
  int32_t max_rows;
  int32_t device;        // -1: validation-only handle (no GPU work is ever enqueued)
  int32_t index_bits;    // ceil(log2(vocab)), at least 1
  int32_t mass_shift;    // fixed-point scale of masses: sum of vocab masses <= 2^62
  void* workspace;       // device memory: split-row counters, then partial results
  uint32_t* split_counter;
  void* split_partials;
  tss::TopPRow* topp_rows;
  tss::TopPCand* topp_list;
  int32_t num_cu;        // compute units of the device (0 for a validation-only handle)
};

namespace {

int ceil_log2(int64_t v) {
  int b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}

// Restores the caller's current device when it goes out of scope.
struct DeviceGuard {
  int saved = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&saved) != hipSuccess) return;
    if (saved == dev) {
      ok = true;
      return;
    }
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (ok && saved >= 0) (void)hipSetDevice(saved);
  }
};

// The logits buffer and row selection of a call.
ts_status check_rows(const ts_sampler* s, const void* logits, ts_dtype dtype,
                     int64_t rows_in_buffer, int64_t row_stride, int32_t n, const int32_t* gather) {
  if (s == nullptr) return TS_E_ARG;
  if (dtype != TS_F32 && dtype != TS_BF16) return TS_E_DTYPE;
  if (n < 0 || rows_in_buffer < 0) return TS_E_ARG;
  if (n > s->max_rows) return TS_E_SIZE;
  if (row_stride < s->vocab) return TS_E_SIZE;
  if (gather == nullptr && rows_in_buffer < n) return TS_E_SIZE;
  if (n == 0) return TS_OK;
  if (logits == nullptr || rows_in_buffer == 0) return TS_E_ARG;
  return TS_OK;
}

ts_status check_common(const ts_sampler* s, const void* logits, ts_dtype dtype,
                       int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                       const int32_t* gather, const int32_t* map, const ts_params* params,
                       int32_t no_top_k, int32_t no_top_p) {
  if (params == nullptr) return TS_E_ARG;
  const ts_status st = check_rows(s, logits, dtype, rows_in_buffer, row_stride, n, gather);
  if (st != TS_OK || n == 0) return st;
  if (params->temperature == nullptr || params->seed == nullptr) return TS_E_ARG;
  if (params->num_requests < 1) return TS_E_ARG;
  if (map == nullptr && params->num_requests < n) return TS_E_SIZE;
  if (!no_top_k && params->top_k == nullptr) return TS_E_ARG;
  if (!no_top_p && params->top_p == nullptr) return TS_E_ARG;
  return TS_OK;
}

tss::RowArgs make_args(const ts_sampler* s, const void* logits, int64_t row_stride, int32_t n,
                       const int32_t* gather, const int32_t* map, const ts_params* p,
                       int32_t no_top_k, int32_t no_top_p) {
  tss::RowArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = s->vocab;
  a.n = n;
  a.gather = gather;
  a.req_map = map;
  a.temperature = p->temperature;
  a.top_k = no_top_k ? nullptr : p->top_k;
  a.top_p = no_top_p ? nullptr : p->top_p;
  a.seed = p->seed;
  a.mass_shift = s->mass_shift;
  a.index_bits = s->index_bits;
  a.split_counter = s->split_counter;
  a.split_partials = s->split_partials;
  a.topp_rows = s->topp_rows;
  a.topp_list = s->topp_list;
  // one fast-kernel workgroup fills a CU: with more rows than CUs the rows
  // that start late should be the quick ones
  a.num_cu = s->num_cu;
  a.heavy_first = (s->num_cu > 0 && n > s->num_cu && n <= 1024) ? 1 : 0;
  return a;
}

}  // namespace

extern "C" {

ts_route ts_select_route(int32_t no_top_k, int32_t no_top_p) {
  if (no_top_k && no_top_p) return TS_ROUTE_NONE;
  if (no_top_p) return TS_ROUTE_TOPK;
  if (no_top_k) return TS_ROUTE_TOPP;
  return TS_ROUTE_JOINT;
}

const char* ts_status_str(ts_status st) {
  switch (st) {
    case TS_OK: return "ok";
    case TS_E_ARG: return "invalid argument";
    case TS_E_DTYPE: return "unsupported logits dtype";
    case TS_E_SIZE: return "size out of range";
    case TS_E_HIP: return "HIP runtime error";
    case TS_E_NOMEM: return "out of device memory";
  }
  return "unknown status";
}

ts_status ts_create(int64_t vocab, int32_t max_rows, int32_t device, ts_sampler** out) {
  if (out == nullptr) return TS_E_ARG;
  *out = nullptr;
  if (vocab < 1 || vocab >= (int64_t(1) << 31) || max_rows < 1 || device < -1) return TS_E_ARG;
  if (device >= 0) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return TS_E_HIP;
  }
  ts_sampler* s = new (std::nothrow) ts_sampler;
  if (s == nullptr) return TS_E_NOMEM;
  s->vocab = vocab;
  s->max_rows = max_rows;
  s->device = device;
  s->index_bits = ceil_log2(vocab) < 1 ? 1 : ceil_log2(vocab);
  const int shift = 62 - ceil_log2(vocab + 1);
  s->mass_shift = shift > 44 ? 44 : shift;
  s->workspace = nullptr;
  s->split_counter = nullptr;
  s->split_partials = nullptr;
  s->topp_rows = nullptr;
  s->topp_list = nullptr;
  s->num_cu = 0;
  if (device >= 0) {
    // counters, padded to 256 bytes, then the partial results, then the
    // per-row top-p state and the top-p cutoff-bucket lists
    const size_t counter_bytes = ((size_t)max_rows * sizeof(uint32_t) + 255) & ~(size_t)255;
    const size_t partial_bytes = (size_t)max_rows * tss::kMaxSplit * sizeof(tss::SplitPartial);
    const size_t topp_bytes = ((size_t)max_rows * sizeof(tss::TopPRow) + 255) & ~(size_t)255;
    const size_t list_bytes = (size_t)max_rows * tss::kTopPListCap * sizeof(tss::TopPCand);
    const size_t bytes = counter_bytes + partial_bytes + topp_bytes + list_bytes;
    DeviceGuard guard(device);
    if (!guard.ok) {
      delete s;
      return TS_E_HIP;
    }
    if (hipDeviceGetAttribute(&s->num_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        s->num_cu < 1) {
      (void)hipGetLastError();
      delete s;
      return TS_E_HIP;
    }
    void* ws = nullptr;
    const hipError_t e = hipMalloc(&ws, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      delete s;
      return e == hipErrorOutOfMemory ? TS_E_NOMEM : TS_E_HIP;
    }
    if (hipMemset(ws, 0, counter_bytes) != hipSuccess) {
      (void)hipFree(ws);
      delete s;
      return TS_E_HIP;
    }
    s->workspace = ws;
    s->split_counter = static_cast<uint32_t*>(ws);
    s->split_partials = static_cast<char*>(ws) + counter_bytes;
    s->topp_rows = reinterpret_cast<tss::TopPRow*>(static_cast<char*>(ws) + counter_bytes + partial_bytes);
    s->topp_list = reinterpret_cast<tss::TopPCand*>(static_cast<char*>(ws) + counter_bytes +
                                                    partial_bytes + topp_bytes);
  }
  *out = s;
  return TS_OK;
}

ts_status ts_destroy(ts_sampler* s) {
  if (s != nullptr && s->workspace != nullptr) {
    DeviceGuard guard(s->device);
    (void)hipFree(s->workspace);
  }
  delete s;
  return TS_OK;
}

ts_status ts_sample(ts_sampler* s, const void* logits, ts_dtype dtype, int64_t rows_in_buffer,
                    int64_t row_stride, int32_t n, const int32_t* gather_indices,
                    const int32_t* token_to_request_index, const ts_params* params,
                    uint64_t step_offset, int32_t no_top_k, int32_t no_top_p, int32_t* out_ids,
                    float* out_logprob, void* stream) {
  ts_status st = check_common(s, logits, dtype, rows_in_buffer, row_stride, n, gather_indices,
                              token_to_request_index, params, no_top_k, no_top_p);
  if (st != TS_OK) return st;
  if (n > 0 && out_ids == nullptr) return TS_E_ARG;
  if (n == 0) return TS_OK;
  if (s->device < 0) return TS_E_HIP;
  DeviceGuard guard(s->device);
  if (!guard.ok) return TS_E_HIP;
  tss::RowArgs a = make_args(s, logits, row_stride, n, gather_indices, token_to_request_index,
                             params, no_top_k, no_top_p);
  a.step_offset = step_offset;
  a.req_offset = params->step_offsets;
  a.out_ids = out_ids;
  a.out_lp = out_logprob;
  const tss::Route route = (tss::Route)ts_select_route(no_top_k, no_top_p);
  const hipError_t err = tss::launch_rows(a, dtype == TS_F32 ? tss::kF32 : tss::kBF16, route,
                                          tss::kOutSample, (hipStream_t)stream);
  return err == hipSuccess ? TS_OK : TS_E_HIP;
}

ts_status ts_log_probs(ts_sampler* s, const void* logits, ts_dtype dtype, int64_t rows_in_buffer,
                       int64_t row_stride, int32_t n, const int32_t* gather_indices,
                       const int32_t* token_to_request_index, const ts_params* params,
                       int32_t no_top_k, int32_t no_top_p, const int32_t* token_ids, float* out,
                       void* stream) {
  ts_status st = check_common(s, logits, dtype, rows_in_buffer, row_stride, n, gather_indices,
                              token_to_request_index, params, no_top_k, no_top_p);
  if (st != TS_OK) return st;
  if (n > 0 && out == nullptr) return TS_E_ARG;
  if (n == 0) return TS_OK;
  if (s->device < 0) return TS_E_HIP;
  DeviceGuard guard(s->device);
  if (!guard.ok) return TS_E_HIP;
  tss::RowArgs a = make_args(s, logits, row_stride, n, gather_indices, token_to_request_index,
                             params, no_top_k, no_top_p);
  a.token_ids = token_ids;
  a.out_lp = out;
  const tss::Route route = (tss::Route)ts_select_route(no_top_k, no_top_p);
  const hipError_t err =
      tss::launch_rows(a, dtype == TS_F32 ? tss::kF32 : tss::kBF16, route,
                       token_ids ? tss::kOutLogProbAt : tss::kOutLogProbFull, (hipStream_t)stream);
  return err == hipSuccess ? TS_OK : TS_E_HIP;
}

ts_status ts_raw_log_probs_at(ts_sampler* s, const void* logits, ts_dtype dtype,
                              int64_t rows_in_buffer, int64_t row_stride, int32_t n,
                              const int32_t* gather_indices, const int32_t* token_ids, float* out,
                              void* stream) {
  ts_status st = check_rows(s, logits, dtype, rows_in_buffer, row_stride, n, gather_indices);
  if (st != TS_OK) return st;
  if (n == 0) return TS_OK;
  if (token_ids == nullptr || out == nullptr) return TS_E_ARG;
  if (s->device < 0) return TS_E_HIP;
  DeviceGuard guard(s->device);
  if (!guard.ok) return TS_E_HIP;
  tss::RowArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = s->vocab;
  a.n = n;
  a.gather = gather_indices;
  a.token_ids = token_ids;
  a.out_lp = out;
  a.split_counter = s->split_counter;
  a.split_partials = s->split_partials;
  if (!tss::split_none_supported(a)) return TS_E_SIZE;
  const hipError_t err = tss::launch_rows_raw_log_prob_at(a, dtype == TS_F32 ? tss::kF32 : tss::kBF16,
                                                          (hipStream_t)stream);
  return err == hipSuccess ? TS_OK : TS_E_HIP;
}

ts_status ts_build_spec_map(int32_t num_decode, int32_t num_prefill, int32_t num_spec,
                            int32_t* out_map, int32_t capacity, int32_t on_device, void* stream,
                            int32_t* out_n) {
  if (num_decode < 0 || num_prefill < 0 || num_spec < 0 || capacity < 0 || out_n == nullptr)
    return TS_E_ARG;
  const int64_t n = (int64_t)num_decode * (1 + (int64_t)num_spec) + num_prefill;
  if (n > 0x7FFFFFFF) return TS_E_SIZE;
  *out_n = (int32_t)n;
  if (n > capacity) return TS_E_SIZE;
  if (n == 0) return TS_OK;
  if (out_map == nullptr) return TS_E_ARG;
  if (!on_device) {
    int64_t row = 0;
    for (int32_t d = 0; d < num_decode; ++d)
      for (int32_t t = 0; t <= num_spec; ++t) out_map[row++] = d;
    for (int32_t i = 0; i < num_prefill; ++i) out_map[row++] = num_decode + i;
    return TS_OK;
  }
  return tss::launch_spec_map(num_decode, num_prefill, num_spec, out_map,
                              (hipStream_t)stream) == hipSuccess
             ? TS_OK
             : TS_E_HIP;
}

ts_status ts_verify_chain(int32_t bs, int32_t n_per_req, const int32_t* candidates,
                          const int32_t* target_sampled, int32_t* predicts, int32_t* accept_index,
                          int32_t* accept_length, void* stream) {
  if (bs < 0 || n_per_req < 1) return TS_E_ARG;
  if ((int64_t)bs * n_per_req > 0x7FFFFFFF) return TS_E_SIZE;
  if (bs == 0) return TS_OK;
  if (candidates == nullptr || target_sampled == nullptr || predicts == nullptr ||
      accept_index == nullptr || accept_length == nullptr)
    return TS_E_ARG;
  return tss::launch_verify_chain(bs, n_per_req, candidates, target_sampled, predicts, accept_index,
                                  accept_length, (hipStream_t)stream) == hipSuccess
             ? TS_OK
             : TS_E_HIP;
}

ts_status ts_check_indices(int32_t n, const int32_t* gather_indices, int64_t rows_in_buffer,
                           const int32_t* token_to_request_index, int32_t num_requests,
                           uint32_t* error_word, void* stream) {
  if (n < 0 || error_word == nullptr) return TS_E_ARG;
  if (gather_indices != nullptr && rows_in_buffer < 1) return TS_E_ARG;
  if (token_to_request_index != nullptr && num_requests < 1) return TS_E_ARG;
  return tss::launch_check_indices(n, gather_indices, rows_in_buffer, token_to_request_index,
                                   num_requests, error_word, (hipStream_t)stream) == hipSuccess
             ? TS_OK
             : TS_E_HIP;
}

}  // extern "C"
