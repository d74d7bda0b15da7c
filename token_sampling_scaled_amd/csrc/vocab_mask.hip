// Vocabulary mask applied to the logits in place.  The TokenSpeed Triton
// sampling backend page calls apply_vocab_mask on the logits after the NaN
// guard and before the greedy or Gumbel step, without printing its body; here
// entry j of a row keeps its logit when bit (j mod 32) of word (j / 32) of the
// row's mask is set, and becomes -inf otherwise, so that no later step of any
// route can select it.
#include "tssample.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kBlock = 256;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// One thread per 16-byte vector of a row (8 bf16 or 4 fp32 entries; EB bytes
// per entry).  A vector whose bits are all set is left alone, one whose bits
// are all clear is overwritten with -inf without being read, the others are
// read, blended and written back.  The vocabulary's last partial vector, and
// every vector of a row that is not 16-byte aligned, go entry by entry.
template <int EB>
__global__ __launch_bounds__(kBlock) void vocab_mask_kernel(char* logits, int64_t rows,
                                                            int64_t row_stride_bytes, int64_t vocab,
                                                            const uint32_t* mask, int64_t mask_stride,
                                                            const int32_t* mask_index) {
  constexpr int kPer = 16 / EB;
  constexpr uint32_t kFull = (1u << kPer) - 1u;
  const int64_t j0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * kPer;
  if (j0 >= vocab) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int64_t mr = mask_index ? (int64_t)mask_index[r] : r;
    // j0 is a multiple of kPer (4 or 8), so the vector's bits lie in one word
    const uint32_t bits = (mask[mr * mask_stride + (j0 >> 5)] >> (uint32_t)(j0 & 31)) & kFull;
    if (bits == kFull) continue;
    char* row = logits + r * row_stride_bytes;
    if (j0 + kPer <= vocab && (reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
      v4u* p = reinterpret_cast<v4u*>(row + j0 * EB);
      v4u out;
      if (EB == 4) {
        const v4u in = bits ? *p : v4u{0u, 0u, 0u, 0u};
#pragma unroll
        for (int d = 0; d < 4; ++d) out[d] = ((bits >> d) & 1u) ? in[d] : 0xFF800000u;
      } else {
        const v4u in = bits ? *p : v4u{0u, 0u, 0u, 0u};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t keep = (((bits >> (2 * d)) & 1u) ? 0x0000FFFFu : 0u) |
                                (((bits >> (2 * d + 1)) & 1u) ? 0xFFFF0000u : 0u);
          out[d] = (in[d] & keep) | (0xFF80FF80u & ~keep);
        }
      }
      *p = out;
    } else {
      for (int e = 0; e < kPer && j0 + e < vocab; ++e) {
        if ((bits >> e) & 1u) continue;
        if (EB == 4)
          reinterpret_cast<uint32_t*>(row)[j0 + e] = 0xFF800000u;
        else
          reinterpret_cast<uint16_t*>(row)[j0 + e] = (uint16_t)0xFF80u;
      }
    }
  }
}

}  // namespace

extern "C" ts_status ts_apply_vocab_mask(int64_t vocab, void* logits, ts_dtype dtype, int64_t rows,
                                         int64_t row_stride, const uint32_t* mask,
                                         int64_t mask_stride_words, const int32_t* mask_index,
                                         void* stream) {
  if (vocab < 1 || vocab >= (int64_t(1) << 31) || rows < 0) return TS_E_ARG;
  if (dtype != TS_F32 && dtype != TS_BF16) return TS_E_DTYPE;
  if (row_stride < vocab || mask_stride_words < (vocab + 31) / 32) return TS_E_SIZE;
  if (rows == 0) return TS_OK;
  if (logits == nullptr || mask == nullptr) return TS_E_ARG;
  const int eb = dtype == TS_F32 ? 4 : 2;
  const int64_t vecs = (vocab * eb + 15) / 16;
  const dim3 grid((uint32_t)((vecs + kBlock - 1) / kBlock), (uint32_t)(rows < 65535 ? rows : 65535));
  const hipStream_t s = (hipStream_t)stream;
  char* base = static_cast<char*>(logits);
  if (eb == 4)
    hipLaunchKernelGGL(vocab_mask_kernel<4>, grid, dim3(kBlock), 0, s, base, rows, row_stride * 4,
                       vocab, mask, mask_stride_words, mask_index);
  else
    hipLaunchKernelGGL(vocab_mask_kernel<2>, grid, dim3(kBlock), 0, s, base, rows, row_stride * 2,
                       vocab, mask, mask_stride_words, mask_index);
  return hipGetLastError() == hipSuccess ? TS_OK : TS_E_HIP;
}
