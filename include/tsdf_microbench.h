/*
 * tsdf_microbench.h -- hardware-ceiling microbenchmarks exported by
 * libtsdf_hip.so.  They measure the rates the integrate kernels are bound
 * by: streaming copy bandwidth (the HBM ceiling and the reference kernel for
 * scaling hardware byte counters), no-return f32 atomic additions and 64-bit
 * compare-exchanges under the access patterns of the update and allocate
 * kernels ("What Irregularity Costs", section 3: five atomic additions per
 * voxel, one compare-exchange per inserted key).  Each call enqueues one
 * kernel on `stream` (a hipStream_t) and returns; the caller times it.
 * Pointers are caller device memory; invalid arguments return TSDF_EINVAL
 * and enqueue nothing.
 */
#ifndef TSDF_MICROBENCH_H
#define TSDF_MICROBENCH_H

#include <stddef.h>
#include <stdint.h>

#include "tsdf.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Access patterns of tsdf_mb_atomic_add_f32 (operation i of n_ops): */
enum {
    TSDF_MB_COALESCED = 0,  /* buf[i mod n]: a wave covers 64 consecutive floats */
    TSDF_MB_RANDOM = 1,     /* buf[hash(i) mod n]: every lane its own cache line */
    TSDF_MB_SAME_WAVE = 2,  /* buf[hash(i / 64) mod n]: a whole wave on one address */
    TSDF_MB_BLOCK_ROW = 3,  /* 64 consecutive floats at a random 512-float block and row */
    TSDF_MB_COUNTERS = 4    /* one lane per wave: counter (wave mod n/32), one 128-byte line each,
                               i.e. n/32 shared counters (contention) */
};

/* dst[0 .. bytes) = src[0 .. bytes); bytes a multiple of 16, both 16-byte aligned. */
tsdf_status tsdf_mb_copy(const void* src, void* dst, size_t bytes, void* stream);

/* n_ops no-return atomic additions of 1.0f into buf[0 .. n), n a power of two
 * (>= 512 for TSDF_MB_BLOCK_ROW, >= 32 for TSDF_MB_COUNTERS, where only one
 * operation in 64 is performed). */
tsdf_status tsdf_mb_atomic_add_f32(float* buf, size_t n, size_t n_ops, int pattern, uint32_t seed, void* stream);

/* n_ops 64-bit compare-exchanges (expected 0, desired op id + 1) at random
 * slots of buf[0 .. n), n a power of two. */
tsdf_status tsdf_mb_cas_u64(uint64_t* buf, size_t n, size_t n_ops, uint32_t seed, void* stream);

/* LDS atomic additions (the owner update sums a block in LDS): operand
 * types and LDS address patterns of tsdf_mb_lds_atomic. */
enum {
    TSDF_MB_LDS_U32 = 0,
    TSDF_MB_LDS_F32 = 1,
    TSDF_MB_LDS_U64 = 2
};
enum {
    TSDF_MB_LDS_DISTINCT = 0,   /* the 64 lanes of a wave on 64 consecutive words */
    TSDF_MB_LDS_RANDOM = 1,     /* every lane a random word of 512 */
    TSDF_MB_LDS_SAME = 2,       /* a whole wave on one word */
    TSDF_MB_LDS_GROUPS = 3      /* groups of 8 lanes on one word */
};

/* n_workgroups workgroups of 256 threads, each thread adding `iters` times
 * into a 512-entry LDS array of the given type with the given pattern.
 * Rate = n_workgroups * 256 * iters lane operations over the kernel time. */
tsdf_status tsdf_mb_lds_atomic(int type, int pattern, uint32_t n_workgroups, uint32_t iters, float* sink,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSDF_MICROBENCH_H */
