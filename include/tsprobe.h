/*
 * tsprobe.h -- C ABI of the measurement probes that ship beside the sampler
 * (libtsprobe.so, gfx950).  They are not part of the sampling path: the
 * benchmark uses them to measure what the hardware allows for the path's own
 * access pattern, and the GPU tests use them to evaluate the device noise
 * transform on its whole domain.
 *
 * Conventions: pointers are device memory of the current HIP device, owned by
 * the caller; "stream" is a hipStream_t (NULL = default stream); calls enqueue
 * work and return; errors come back as an int status (0 ok, 1 invalid
 * argument, 4 HIP launch error), never thrown.
 */
#ifndef TSPROBE_H
#define TSPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming-read ceiling: reads `rows` rows of `row_bytes` bytes each (rows
 * `row_stride_bytes` apart, both multiples of 16, data 16-byte aligned) with
 * the launch shape of the register-resident sampling kernel -- one workgroup of
 * 1024 threads per row, each thread issuing `loads_per_thread` non-temporal
 * 16-byte loads (1, 2, 4, 8 or 16; row_bytes <= 16384 * loads_per_thread) --
 * and writes the xor of each row's words to out[row] (device uint32 [rows]), so
 * no load can be dropped.  The time of one call over bytes that are not in
 * any cache is the most a kernel of this shape can read per second, the
 * ceiling reported beside the 8 TB/s HBM peak.  Errors: 1 (rows < 1, sizes
 * not multiples of 16, too many bytes for the shape, NULL pointers), 4. */
int tsp_read_rows(const void* data, int64_t rows, int64_t row_bytes, int64_t row_stride_bytes,
                  int32_t loads_per_thread, uint32_t* out, void* stream);

/* Streaming read of rows of any length: `parts` workgroups of `threads`
 * (256, 512 or 1024) threads per row, each reading its share of the row's
 * 16-byte vectors with a ring of 16 loads in flight per thread, non-temporal
 * when `nontemporal` is nonzero.  out[row] (device uint32 [rows], zeroed by
 * the caller) receives the xor of the row's words, so no load can be
 * dropped.  The time of one call is the read ceiling of that launch shape
 * (for the top-p route's one workgroup of 1024 threads per row, among
 * others).  Errors: 1 (sizes not multiples of 16, bad shape, NULL), 4. */
int tsp_read_rows_ring(const void* data, int64_t rows, int64_t row_bytes, int64_t row_stride_bytes,
                       int32_t threads, int32_t parts, int32_t nontemporal, uint32_t* out,
                       void* stream);

/* An empty kernel of `blocks` workgroups of 1024 threads: the launch and
 * drain cost any one-launch call pays.  Errors: 1 (blocks < 1), 4. */
int tsp_empty(int32_t blocks, void* stream);

/* Noise throughput: `blocks` workgroups of 256 threads, each thread drawing
 * `per_thread` Philox4x32-10 blocks (counter (i, thread, 0x5EED, 0), a fixed
 * key) with the sampling kernels' own generator; with with_gumbel != 0 every
 * word also goes through the base-2 Gumbel transform and the thread keeps the
 * largest, as the draw kernels do.  blocks * 256 * per_thread / (time of one
 * call) is the device's rate of noise blocks: the arithmetic bound of a
 * kernel that draws noise for most of a row.  out: device uint32 [blocks *
 * 256], written (what each thread kept).  Errors: 1 (blocks < 1,
 * per_thread < 1, too many threads, NULL), 4. */
int tsp_noise_rate(int32_t blocks, int32_t per_thread, int32_t with_gumbel, uint32_t* out,
                   void* stream);

/* The device's integer -> Gumbel noise transforms, evaluated on every one of
 * the 2^23 uniforms u_i = (i + 1/2) 2^-23 they can see (word w = i << 9):
 *   g[i]  = the natural-log Gumbel variate -ln(-ln u_i) as the sampling
 *           kernels compute it (device float),
 *   g2[i] = the base-2 form -log2(-log2 u_i) that the split and top-p kernels
 *           race in base-2 units.
 * g and g2 are device float [2^23] each, written.  Errors: 1 (NULL), 4. */
int tsp_gumbel_table(float* g, float* g2, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSPROBE_H */
