/*
 * moe_measure.h — measurement helpers, built as their own library
 * (libmoe_measure.so) apart from the layer's.  Nothing here is a step of the
 * MoE layer; the benchmark uses it to find the practical bandwidth ceiling the
 * layer's bandwidth-bound kernels are compared with.
 */
#ifndef MOE_MEASURE_H
#define MOE_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* moe_measure_hbm_read — enqueue one plain streaming read of `bytes` bytes at
 * `src` (device, 16-byte aligned, bytes a multiple of 16) by `grid`
 * workgroups of 256 threads (1 <= grid <= 65536) on `stream` (a hipStream_t,
 * NULL = null stream).  Each thread writes the XOR fold of the 32-bit words
 * it read to sink[block*256 + thread] (device, grid*256 uint32, caller-owned),
 * so the XOR of all of sink equals the XOR of every word of the region.
 * Returns 0, 1 for invalid arguments (nothing enqueued), or 3 when the launch
 * failed.  Allocates nothing. */
int moe_measure_hbm_read(const void* src, int64_t bytes, int32_t grid, uint32_t* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MEASURE_H */
