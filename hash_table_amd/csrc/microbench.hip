// microbench.hip -- ceilings for the integrate kernels: copy bandwidth,
// float atomic-add rate by access pattern, 64-bit compare-exchange rate,
// LDS atomic-add rate by operand type and pattern.
#include <hip/hip_runtime.h>

#include "tsdf_microbench.h"

namespace {

constexpr int kThreads = 256;
constexpr unsigned int kMaxGrid = 16384;

__device__ __forceinline__ unsigned int mix32(unsigned int x) {   // integer hash (lowbias32)
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(kThreads) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    unsigned long long n) {
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (unsigned long long)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void k_atomic_add(float* buf, unsigned long long mask, unsigned long long n_ops,
                                                          int pattern, unsigned int seed) {
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_ops;
         i += (unsigned long long)gridDim.x * blockDim.x) {
        unsigned long long a;
        switch (pattern) {
            case 0: a = i & mask; break;
            case 1: a = mix32((unsigned int)i ^ seed) & mask; break;
            case 2: a = mix32((unsigned int)(i >> 6) ^ seed) & mask; break;
            case 3: {
                const unsigned int h = mix32((unsigned int)(i >> 6) ^ seed);
                a = (((unsigned long long)(h >> 3) * 512ull + (h & 7u) * 64ull) & mask & ~63ull) + (i & 63);
                break;
            }
            default:       // one lane per wave, on one of n / 32 counters (a 128-byte line each)
                if (i & 63) continue;
                a = ((i >> 6) * 32ull) & mask;
        }
        unsafeAtomicAdd(buf + a, 1.0f);
    }
}

__global__ __launch_bounds__(kThreads) void k_cas(unsigned long long* buf, unsigned long long mask,
                                                   unsigned long long n_ops, unsigned int seed) {
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_ops;
         i += (unsigned long long)gridDim.x * blockDim.x)
        atomicCAS(buf + (mix32((unsigned int)i ^ seed) & mask), 0ull, i + 1);
}

template <int TYPE, int PAT>
__global__ __launch_bounds__(kThreads) void k_lds_atomic(unsigned int iters, float* sink) {
    __shared__ unsigned int au[512];
    __shared__ float af[512];
    __shared__ unsigned long long a64[512];
    for (int i = threadIdx.x; i < 512; i += kThreads) {
        au[i] = 0;
        af[i] = 0.0f;
        a64[i] = 0;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned int x = mix32(threadIdx.x * 2654435761u ^ blockIdx.x);
    for (unsigned int it = 0; it < iters; ++it) {
        int j;
        if (PAT == 0) {
            j = (lane + 64 * wave + (int)it) & 511;
        } else if (PAT == 1) {
            x = x * 1664525u + 1013904223u;
            j = (int)((x >> 8) & 511u);
        } else if (PAT == 2) {
            j = ((int)it * 7 + wave) & 511;
        } else {
            j = ((lane >> 3) * 9 + (int)it + 64 * wave) & 511;
        }
        if (TYPE == 0) atomicAdd(&au[j], 1u);
        else if (TYPE == 1) atomicAdd(&af[j], 1.0f);
        else atomicAdd(&a64[j], 1ull);
    }
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)au[5] + af[7] + (float)a64[9];
}

template <int TYPE>
void launch_lds(int pattern, unsigned int grid, unsigned int iters, float* sink, hipStream_t s) {
    switch (pattern) {
        case 0: hipLaunchKernelGGL((k_lds_atomic<TYPE, 0>), dim3(grid), dim3(kThreads), 0, s, iters, sink); break;
        case 1: hipLaunchKernelGGL((k_lds_atomic<TYPE, 1>), dim3(grid), dim3(kThreads), 0, s, iters, sink); break;
        case 2: hipLaunchKernelGGL((k_lds_atomic<TYPE, 2>), dim3(grid), dim3(kThreads), 0, s, iters, sink); break;
        default: hipLaunchKernelGGL((k_lds_atomic<TYPE, 3>), dim3(grid), dim3(kThreads), 0, s, iters, sink);
    }
}

unsigned int grid_for(unsigned long long n) {
    unsigned long long g = (n + kThreads - 1) / kThreads;
    return (unsigned int)(g < 1 ? 1 : (g > kMaxGrid ? kMaxGrid : g));
}

bool pow2(size_t n) { return n && !(n & (n - 1)); }

tsdf_status launched() { return hipGetLastError() == hipSuccess ? TSDF_OK : TSDF_EHIP; }

}  // namespace

extern "C" {

tsdf_status tsdf_mb_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return TSDF_EINVAL;
    if (!bytes) return TSDF_OK;
    const unsigned long long n = bytes / 16;
    hipLaunchKernelGGL(k_copy, dim3(grid_for(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
    return launched();
}

tsdf_status tsdf_mb_atomic_add_f32(float* buf, size_t n, size_t n_ops, int pattern, uint32_t seed, void* stream) {
    if (!buf || !pow2(n) || pattern < 0 || pattern > 4 || (pattern == 3 && n < 512) || (pattern == 4 && n < 32))
        return TSDF_EINVAL;
    if (!n_ops) return TSDF_OK;
    hipLaunchKernelGGL(k_atomic_add, dim3(grid_for(n_ops)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), buf,
                       (unsigned long long)(n - 1), (unsigned long long)n_ops, pattern, seed);
    return launched();
}

tsdf_status tsdf_mb_cas_u64(uint64_t* buf, size_t n, size_t n_ops, uint32_t seed, void* stream) {
    if (!buf || !pow2(n)) return TSDF_EINVAL;
    if (!n_ops) return TSDF_OK;
    hipLaunchKernelGGL(k_cas, dim3(grid_for(n_ops)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<unsigned long long*>(buf), (unsigned long long)(n - 1),
                       (unsigned long long)n_ops, seed);
    return launched();
}

tsdf_status tsdf_mb_lds_atomic(int type, int pattern, uint32_t n_workgroups, uint32_t iters, float* sink,
                               void* stream) {
    if (!sink || type < 0 || type > 2 || pattern < 0 || pattern > 3 || n_workgroups < 1 || n_workgroups > kMaxGrid)
        return TSDF_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (type == 0) launch_lds<0>(pattern, n_workgroups, iters, sink, s);
    else if (type == 1) launch_lds<1>(pattern, n_workgroups, iters, sink, s);
    else launch_lds<2>(pattern, n_workgroups, iters, sink, s);
    return launched();
}

}  // extern "C"
