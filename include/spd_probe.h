/*
 * spd_probe.h -- C ABI of libspd_probe.so: measurement kernels that bound the
 * attention path from below, for the benchmark.  They are not part of the
 * attention path and compute nothing a caller uses.
 *
 *   spd_probe_gather: the row gather of the attention kernels alone -- the
 *     same ragged CSR slices (sglang PR #28392 summary page, "key source
 *     snippet": token t reads pool rows kv_indices[kv_indptr[t] :
 *     kv_indptr[t+1]], each D bf16 values), staged into LDS by the same
 *     LDS-DMA loads, 16-row tiles, four waves taking every fourth tile, two
 *     tiles in flight a wave -- with no arithmetic.  A workgroup takes
 *     (token, group, partition): `groups` workgroups read every row of a
 *     token (as head groups do), `parts` split its rows into equal shares
 *     (as split-L partitions do).
 *   spd_probe_null: an empty kernel of `workgroups` x 256 threads (the
 *     launch and drain of one kernel).
 *   spd_probe_store: `workgroups` x 256 threads store `bytes` of zeros (an
 *     output written by the whole grid at once).
 *
 * All calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream), allocate nothing and return 0 on success, 1 for invalid arguments
 * (checked on the host before any HIP call), 4 when a launch fails.
 * Caller preconditions (not checked): every index lies in [0, num_rows) of
 * the pool, kv_indptr is non-decreasing from 0.
 */
#ifndef SPD_PROBE_H_
#define SPD_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPD_PROBE_API __attribute__((visibility("default")))

/*
 *   kv           [num_rows, D] bf16 pool, 16-byte aligned
 *   kv_indices   int32 row indices, kv_indptr [N+1] int32 (device)
 *   D            64, 128, 256 or 512
 *   groups, parts >= 1; N * groups * parts < 2^31 workgroups
 *   out_words    [N * groups * parts] uint32 (device): one LDS word per
 *                workgroup, so the loads have a consumer
 */
SPD_PROBE_API int spd_probe_gather(const void* kv, const int32_t* kv_indices,
                                   const int32_t* kv_indptr, int32_t N, int32_t D, int32_t groups,
                                   int32_t parts, uint32_t* out_words, void* stream);

SPD_PROBE_API int spd_probe_null(int32_t workgroups, void* stream);

/* out: device buffer of `bytes` (a multiple of 16, 16-byte aligned) */
SPD_PROBE_API int spd_probe_store(void* out, int64_t bytes, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPD_PROBE_H_ */
