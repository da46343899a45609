/*
 * kda_calib.h -- C ABI of libkda_calib.so: streaming kernels of known byte
 * counts for measurement.  They are not part of the mixer and no passage of the
 * pages defines them; the benchmark uses them to measure the HBM ceiling of an
 * access pattern and to calibrate the hardware byte counters against kernels
 * whose traffic is known exactly.
 *
 * Pointers are device pointers owned by the caller; nothing is allocated or
 * synchronised; work is enqueued on `stream`.  Return value: 0 on success,
 * 1 for an invalid argument (NULL, misaligned, size not a multiple of 16 B),
 * 3 when the launch fails.
 */
#ifndef KDA_CALIB_H_
#define KDA_CALIB_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In-place read-modify-write of `num_states` fp32 128 x 128 states (64 KiB each,
 * 16-byte aligned): every value is multiplied by `scale`.  One workgroup of 512
 * threads per state with the decode kernel's mapping (thread t reads columns
 * 4 (t % 32) .. +3 of rows t / 32 + 16 m, m = 0..7, non-temporal): reads and
 * writes exactly 65,536 B per state. */
int kda_calib_state_rmw(void *state, int64_t num_states, float scale, hipStream_t stream);

/* dst = src over `bytes` (a multiple of 16; both 16-byte aligned, not
 * overlapping): reads `bytes` and writes `bytes`. */
int kda_calib_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

/* Every fp32 value of dst (`bytes`, a multiple of 16, 16-byte aligned) set to
 * `value`: writes `bytes`, reads nothing. */
int kda_calib_fill(void *dst, size_t bytes, float value, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_CALIB_H_ */
