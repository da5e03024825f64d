// tsdf.hip -- kernels and C ABI of libtsdf_hip.so (gfx950).
//
// The integrate path of hash-blocked TSDF fusion as "What Irregularity
// Costs: CUDA C++, Rust, and Triton on a Hash-Blocked GPU Workload"
// describes it in section 3: two kernels over the same points, `allocate`
// (the irregular stage: probe, compare-exchange, insert) and `update` (the
// regular stage: look up, five atomic additions per voxel).  Both apply the
// same occlusion test.  Memory is the caller's (section 3a: allocated once
// by the harness, handed over through a C ABI).
//
// Launch geometry: one thread per pixel; a 256-thread workgroup (four wave64
// wavefronts) covers a 16 x 16 pixel tile, each wavefront an 8 x 8 sub-tile,
// so the 64 lanes of a wave walk neighbouring rays that mostly touch the
// same blocks and the same pool cache lines.  Workgroups are dispatched to
// the eight XCDs round-robin; the workgroup -> tile remap gives each XCD a
// contiguous run of tiles so neighbouring tiles share an L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/tsdf.h"
#include "tsdf_device.hpp"

using namespace tsdf;

namespace {

constexpr int kTile = 16;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// pixel of this thread, from the remapped tile; false if the workgroup has
// no tile (grid rounded up to a multiple of 8) -- uniform per workgroup
__device__ __forceinline__ bool workgroup_tile(const FrameArgs& f, int& tile_u0, int& tile_v0) {
    const int wg = blockIdx.x;
    const int tile = (wg % kXcds) * f.tiles_per_xcd + wg / kXcds;
    if (tile >= f.n_tiles) return false;
    tile_u0 = (tile % f.tiles_x) * kTile;
    tile_v0 = (tile / f.tiles_x) * kTile;
    return true;
}

__device__ __forceinline__ void thread_pixel(int tile_u0, int tile_v0, int& u, int& v) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    u = tile_u0 + (wave & 1) * 8 + (lane & 7);
    v = tile_v0 + (wave >> 1) * 8 + (lane >> 3);
}

__device__ __forceinline__ void hist_add(unsigned int* s_hist, unsigned int* s_pmax, unsigned int probes) {
    atomicAdd(s_hist + (probes < (unsigned)kProbeBins ? probes - 1 : kProbeBins - 1), 1u);
    atomicMax(s_pmax, probes);
}

__device__ __forceinline__ void flush_hist(const unsigned int* s_hist, const unsigned int* s_pmax,
                                           unsigned long long* counters, int base) {
    const int t = threadIdx.x;
    if (t < kProbeBins && s_hist[t]) atomicAdd(counters + base + t, (unsigned long long)s_hist[t]);
    if (t == kProbeBins && *s_pmax) atomicMax(counters + kProbeMax, (unsigned long long)*s_pmax);
}

// ---------------------------------------------------------------------------
// allocate: walk, test, and insert each new block key of the ray.  Keys are
// de-duplicated within the wavefront before probing: at each step the lanes
// that entered a new block elect one leader per distinct key (ballot loop),
// and only leaders probe, concurrently.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_allocate(FrameArgs f, VolumeArgs vol) {
    __shared__ unsigned int s_hist[kProbeBins];
    __shared__ unsigned int s_pmax;
    __shared__ unsigned int s_guard;
    int tu, tv;
    if (!workgroup_tile(f, tu, tv)) return;
    if (threadIdx.x < kProbeBins) s_hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        s_pmax = 0;
        s_guard = 0;
    }
    __syncthreads();

    int u, v;
    thread_pixel(tu, tv, u, v);
    BandWalk w;
    bool alive = false;
    if (u < f.width && v < f.height) {
        const float d = f.depth[(size_t)v * f.width + u];
        alive = setup_walk(w, d, u, v, f, vol.trunc, vol.inv_vs) == kValid;
    }
    const int lane = threadIdx.x & 63;
    unsigned long long cur = kEmptyKey;
    int visits = 0;
    unsigned int guard_hits = 0;
    while (__any(alive)) {
        bool need = false;
        unsigned long long key = kEmptyKey;
        if (alive) {
            float sdf;
            if (centre_test(w, f, vol.vs, vol.trunc, sdf)) {
                key = block_key(w.k0, w.k1, w.k2);
                if (key != cur) {
                    need = true;
                    cur = key;
                }
            }
            if (++visits >= f.max_visits) {
                guard_hits += advance(w) ? 1u : 0u;
                alive = false;
            } else {
                alive = advance(w);
            }
        }
        // one leader per distinct key among the lanes that need an insert
        unsigned long long pending = __ballot(need);
        bool leader = false;
        while (pending) {
            const int l = __ffsll((long long)pending) - 1;
            const unsigned long long lk = __shfl(key, l, 64);
            const bool same = need && key == lk;
            leader |= same && lane == l;
            pending &= ~__ballot(same);
        }
        if (leader) hist_add(s_hist, &s_pmax, insert_key(vol, key));
    }
    if (guard_hits) atomicAdd(&s_guard, guard_hits);
    __syncthreads();
    flush_hist(s_hist, &s_pmax, vol.counters, kHistAlloc);
    if (threadIdx.x == 0 && s_guard) atomicAdd(vol.counters + kWalkGuard, (unsigned long long)s_guard);
}

// ---------------------------------------------------------------------------
// update: walk, test, look the block up once per block run of the ray, and
// add the contribution with five no-return float atomics into the
// structure-of-arrays pool.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_update(FrameArgs f, VolumeArgs vol) {
    __shared__ unsigned int s_hist[kProbeBins];
    __shared__ unsigned int s_pmax;
    __shared__ unsigned int s_cnt[6];
    int tu, tv;
    if (!workgroup_tile(f, tu, tv)) return;
    if (threadIdx.x < kProbeBins) s_hist[threadIdx.x] = 0;
    if (threadIdx.x < 6) s_cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0) s_pmax = 0;
    __syncthreads();

    int u, v;
    thread_pixel(tu, tv, u, v);
    BandWalk w;
    int cls = kInvalid;
    float cr = 0.f, cg = 0.f, cb = 0.f;
    if (u < f.width && v < f.height) {
        const size_t pix = (size_t)v * f.width + u;
        cls = setup_walk(w, f.depth[pix], u, v, f, vol.trunc, vol.inv_vs);
        if (cls == kValid) {
            const float s = 1.0f / 255.0f;
            cr = (float)f.rgb[3 * pix + 0] * s;
            cg = (float)f.rgb[3 * pix + 1] * s;
            cb = (float)f.rgb[3 * pix + 2] * s;
        }
    }
    unsigned int n_updates = 0, n_miss = 0, n_guard = 0;
    if (cls == kValid) {
        unsigned long long cur = kEmptyKey;
        unsigned int idx = kNoIndex;
        int visits = 0;
        for (;;) {
            float sdf;
            if (centre_test(w, f, vol.vs, vol.trunc, sdf)) {
                const unsigned long long key = block_key(w.k0, w.k1, w.k2);
                if (key != cur) {
                    unsigned int probes;
                    idx = lookup_key(vol, key, probes);
                    cur = key;
                    hist_add(s_hist, &s_pmax, probes);
                }
                ++n_updates;
                if (idx != kNoIndex) {
                    const size_t off = (size_t)idx * kBlockVoxels + voxel_in_block(w.k0, w.k1, w.k2);
                    unsafeAtomicAdd(vol.tsdf + off, sdf * vol.inv_trunc);
                    unsafeAtomicAdd(vol.weight + off, 1.0f);
                    unsafeAtomicAdd(vol.r + off, cr);
                    unsafeAtomicAdd(vol.g + off, cg);
                    unsafeAtomicAdd(vol.b + off, cb);
                } else {
                    ++n_miss;
                }
            }
            if (++visits >= f.max_visits) {
                n_guard += advance(w) ? 1u : 0u;
                break;
            }
            if (!advance(w)) break;
        }
    }
    // per-wave sums, then one LDS add per wave, then one global add per counter
    const unsigned int c_valid = wave_sum(cls == kValid);
    const unsigned int c_near = wave_sum(cls == kNear);
    const unsigned int c_oor = wave_sum(cls == kOutside);
    const unsigned int c_upd = wave_sum(n_updates);
    const unsigned int c_miss = wave_sum(n_miss);
    const unsigned int c_guard = wave_sum(n_guard);
    if ((threadIdx.x & 63) == 0) {
        if (c_valid) atomicAdd(s_cnt + 0, c_valid);
        if (c_near) atomicAdd(s_cnt + 1, c_near);
        if (c_oor) atomicAdd(s_cnt + 2, c_oor);
        if (c_upd) atomicAdd(s_cnt + 3, c_upd);
        if (c_miss) atomicAdd(s_cnt + 4, c_miss);
        if (c_guard) atomicAdd(s_cnt + 5, c_guard);
    }
    __syncthreads();
    flush_hist(s_hist, &s_pmax, vol.counters, kHistUpdate);
    if (threadIdx.x == 0) {
        if (s_cnt[0]) atomicAdd(vol.counters + kPointsValid, (unsigned long long)s_cnt[0]);
        if (s_cnt[1]) atomicAdd(vol.counters + kNearSkipped, (unsigned long long)s_cnt[1]);
        if (s_cnt[2]) atomicAdd(vol.counters + kOutOfRange, (unsigned long long)s_cnt[2]);
        if (s_cnt[3]) atomicAdd(vol.counters + kVoxelUpdates, (unsigned long long)s_cnt[3]);
        if (s_cnt[4]) atomicAdd(vol.counters + kUpdateMisses, (unsigned long long)s_cnt[4]);
        if (s_cnt[5]) atomicAdd(vol.counters + kWalkGuard, (unsigned long long)s_cnt[5]);
    }
}

// ---------------------------------------------------------------------------
// initialisation, reset and export
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_fill_table(uint4* table, unsigned long long n) {
    const uint4 empty = make_uint4(~0u, ~0u, ~0u, ~0u);
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (unsigned long long)gridDim.x * blockDim.x)
        table[i] = empty;
}

// Zero the first `blocks` pool blocks of all five arrays; with use_counter,
// only min(block counter, capacity) blocks (the used part).
__global__ __launch_bounds__(kThreads) void k_zero_pool(float4* a0, float4* a1, float4* a2, float4* a3,
                                                         float4* a4, const unsigned long long* counters,
                                                         unsigned long long capacity, int use_counter) {
    unsigned long long blocks = capacity;
    if (use_counter) {
        const unsigned long long used = counters[kBlockCounter];
        blocks = used < capacity ? used : capacity;
    }
    const unsigned long long n = blocks * (kBlockVoxels / 4);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (unsigned long long)gridDim.x * blockDim.x) {
        a0[i] = z;
        a1[i] = z;
        a2[i] = z;
        a3[i] = z;
        a4[i] = z;
    }
}

__global__ __launch_bounds__(kThreads) void k_zero_counters(unsigned long long* counters) {
    for (int i = threadIdx.x; i < kCounterWords; i += blockDim.x) counters[i] = 0;
}

__global__ __launch_bounds__(kThreads) void k_export_coords(const Entry* table, unsigned long long n_entries,
                                                             unsigned long long n_blocks, int* coords) {
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_entries;
         i += (unsigned long long)gridDim.x * blockDim.x) {
        const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(table + i);
        const unsigned int idx = (unsigned int)e.y;
        if (e.x == kEmptyKey || idx >= n_blocks) continue;
        coords[3 * (size_t)idx + 0] = (int)(e.x & 0x1FFFFFull) - kKeyBias;
        coords[3 * (size_t)idx + 1] = (int)((e.x >> 21) & 0x1FFFFFull) - kKeyBias;
        coords[3 * (size_t)idx + 2] = (int)((e.x >> 42) & 0x1FFFFFull) - kKeyBias;
    }
}

unsigned int grid_for(unsigned long long n) {
    unsigned long long g = (n + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > 8192) g = 8192;
    return (unsigned int)g;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
struct tsdf_volume {
    tsdf_config cfg;
    tsdf_buffers buf;
    unsigned int mask;
};

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

VolumeArgs volume_args(const tsdf_volume* h) {
    VolumeArgs a;
    a.table = static_cast<Entry*>(h->buf.table);
    a.mask = h->mask;
    a.capacity = (unsigned long long)h->cfg.pool_capacity;
    a.tsdf = h->buf.tsdf;
    a.weight = h->buf.weight;
    a.r = h->buf.r;
    a.g = h->buf.g;
    a.b = h->buf.b;
    a.counters = static_cast<unsigned long long*>(h->buf.counters);
    a.vs = h->cfg.voxel_size;
    a.inv_vs = 1.0f / h->cfg.voxel_size;
    a.trunc = h->cfg.trunc;
    a.inv_trunc = 1.0f / h->cfg.trunc;
    return a;
}

// Validate a frame and fill the launch arguments.  Returns TSDF_OK, or
// TSDF_EINVAL; *empty is set for a frame without pixels.
tsdf_status frame_args(const tsdf_volume* h, const tsdf_frame* fr, bool need_rgb, FrameArgs* a, bool* empty) {
    if (!fr) return TSDF_EINVAL;
    if (fr->width < 0 || fr->height < 0) return TSDF_EINVAL;
    const int64_t pixels = (int64_t)fr->width * fr->height;
    if (pixels > (int64_t)1 << 31) return TSDF_EINVAL;
    *empty = pixels == 0;
    if (*empty) return TSDF_OK;
    if (!fr->depth || (need_rgb && !fr->rgb)) return TSDF_EINVAL;
    if (!std::isfinite(fr->fx) || !std::isfinite(fr->fy) || fr->fx == 0.0f || fr->fy == 0.0f) return TSDF_EINVAL;
    if (!std::isfinite(fr->cx) || !std::isfinite(fr->cy)) return TSDF_EINVAL;
    for (int i = 0; i < 9; ++i)
        if (!std::isfinite(fr->R[i])) return TSDF_EINVAL;
    for (int i = 0; i < 3; ++i)
        if (!std::isfinite(fr->t[i])) return TSDF_EINVAL;
    // Bound on the cells one walk can visit: 1 + (crossings per axis <=
    // |extent| + 2), extent_i = sum_j |R_ij| |b_j - a_j| / vs with
    // |b - a| = 2 trunc (|xn|, |yn|, 1) at the image corners; + 8 of slack.
    const double mx = std::max(std::fabs(0.0 - fr->cx), std::fabs(fr->width - 1.0 - fr->cx)) / std::fabs(fr->fx);
    const double my = std::max(std::fabs(0.0 - fr->cy), std::fabs(fr->height - 1.0 - fr->cy)) / std::fabs(fr->fy);
    const double span[3] = {mx, my, 1.0};
    double bound = 1.0 + 6.0 + 8.0;
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            bound += std::fabs((double)fr->R[3 * i + j]) * 2.0 * h->cfg.trunc * span[j] / h->cfg.voxel_size;
    if (!(bound <= TSDF_MAX_WALK)) return TSDF_EINVAL;

    a->depth = fr->depth;
    a->rgb = fr->rgb;
    a->width = fr->width;
    a->height = fr->height;
    a->fx = fr->fx;
    a->fy = fr->fy;
    a->cx = fr->cx;
    a->cy = fr->cy;
    std::memcpy(a->R, fr->R, sizeof(a->R));
    std::memcpy(a->t, fr->t, sizeof(a->t));
    a->max_visits = (int)std::ceil(bound);
    a->tiles_x = (fr->width + kTile - 1) / kTile;
    const int tiles_y = (fr->height + kTile - 1) / kTile;
    a->n_tiles = a->tiles_x * tiles_y;
    a->tiles_per_xcd = (a->n_tiles + kXcds - 1) / kXcds;
    return TSDF_OK;
}

tsdf_status launched() { return hipGetLastError() == hipSuccess ? TSDF_OK : TSDF_EHIP; }

}  // namespace

extern "C" {

int64_t tsdf_table_entries_for(int64_t pool_capacity) {
    if (pool_capacity < 1 || pool_capacity > TSDF_MAX_POOL_BLOCKS) return -1;
    int64_t t = 1;
    while (t < 2 * pool_capacity) t <<= 1;
    return t;
}

size_t tsdf_counters_bytes(void) { return sizeof(unsigned long long) * kCounterWords; }

tsdf_status tsdf_create(const tsdf_config* config, const tsdf_buffers* buffers, void* stream, tsdf_volume** out) {
    if (!config || !buffers || !out) return TSDF_EINVAL;
    *out = nullptr;
    if (!finite_pos(config->voxel_size) || !finite_pos(config->trunc)) return TSDF_EINVAL;
    if (config->pool_capacity < 1 || config->pool_capacity > TSDF_MAX_POOL_BLOCKS) return TSDF_EINVAL;
    int64_t entries = config->table_entries;
    if (entries == 0) entries = tsdf_table_entries_for(config->pool_capacity);
    if (!is_pow2(entries) || entries < 2 * config->pool_capacity || entries > TSDF_MAX_TABLE_ENTRIES)
        return TSDF_EINVAL;
    const tsdf_buffers& b = *buffers;
    if (!b.table || !b.tsdf || !b.weight || !b.r || !b.g || !b.b || !b.counters) return TSDF_EINVAL;
    if (!aligned16(b.table) || !aligned16(b.tsdf) || !aligned16(b.weight) || !aligned16(b.r) ||
        !aligned16(b.g) || !aligned16(b.b) || !aligned16(b.counters))
        return TSDF_EALIGN;

    tsdf_volume* h = new (std::nothrow) tsdf_volume;
    if (!h) return TSDF_EINVAL;
    h->cfg = *config;
    h->cfg.table_entries = entries;
    h->buf = b;
    h->mask = (unsigned int)(entries - 1);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned long long cap = (unsigned long long)config->pool_capacity;
    hipLaunchKernelGGL(k_zero_pool, dim3(grid_for(cap * (kBlockVoxels / 4))), dim3(kThreads), 0, s,
                       (float4*)b.tsdf, (float4*)b.weight, (float4*)b.r, (float4*)b.g, (float4*)b.b,
                       (const unsigned long long*)b.counters, cap, 0);
    hipLaunchKernelGGL(k_fill_table, dim3(grid_for((unsigned long long)entries)), dim3(kThreads), 0, s,
                       (uint4*)b.table, (unsigned long long)entries);
    hipLaunchKernelGGL(k_zero_counters, dim3(1), dim3(kThreads), 0, s, (unsigned long long*)b.counters);
    if (launched() != TSDF_OK) {
        delete h;
        return TSDF_EHIP;
    }
    *out = h;
    return TSDF_OK;
}

tsdf_status tsdf_reset(tsdf_volume* h, void* stream) {
    if (!h) return TSDF_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const tsdf_buffers& b = h->buf;
    const unsigned long long cap = (unsigned long long)h->cfg.pool_capacity;
    // the pool clear reads the block counter, so it runs before the counters are cleared
    hipLaunchKernelGGL(k_zero_pool, dim3(grid_for(cap * (kBlockVoxels / 4))), dim3(kThreads), 0, s,
                       (float4*)b.tsdf, (float4*)b.weight, (float4*)b.r, (float4*)b.g, (float4*)b.b,
                       (const unsigned long long*)b.counters, cap, 1);
    hipLaunchKernelGGL(k_fill_table, dim3(grid_for((unsigned long long)h->cfg.table_entries)), dim3(kThreads), 0,
                       s, (uint4*)b.table, (unsigned long long)h->cfg.table_entries);
    hipLaunchKernelGGL(k_zero_counters, dim3(1), dim3(kThreads), 0, s, (unsigned long long*)b.counters);
    return launched();
}

tsdf_status tsdf_allocate(tsdf_volume* h, const tsdf_frame* frame, void* stream) {
    if (!h) return TSDF_EINVAL;
    FrameArgs fa;
    bool empty = false;
    const tsdf_status st = frame_args(h, frame, false, &fa, &empty);
    if (st != TSDF_OK || empty) return st;
    hipLaunchKernelGGL(k_allocate, dim3(fa.tiles_per_xcd * kXcds), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), fa, volume_args(h));
    return launched();
}

tsdf_status tsdf_update(tsdf_volume* h, const tsdf_frame* frame, void* stream) {
    if (!h) return TSDF_EINVAL;
    FrameArgs fa;
    bool empty = false;
    const tsdf_status st = frame_args(h, frame, true, &fa, &empty);
    if (st != TSDF_OK || empty) return st;
    hipLaunchKernelGGL(k_update, dim3(fa.tiles_per_xcd * kXcds), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), fa, volume_args(h));
    return launched();
}

tsdf_status tsdf_integrate(tsdf_volume* h, const tsdf_frame* frame, void* stream) {
    if (!h) return TSDF_EINVAL;
    FrameArgs fa;
    bool empty = false;
    const tsdf_status st = frame_args(h, frame, true, &fa, &empty);
    if (st != TSDF_OK || empty) return st;
    const VolumeArgs va = volume_args(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_allocate, dim3(fa.tiles_per_xcd * kXcds), dim3(kThreads), 0, s, fa, va);
    hipLaunchKernelGGL(k_update, dim3(fa.tiles_per_xcd * kXcds), dim3(kThreads), 0, s, fa, va);
    return launched();
}

tsdf_status tsdf_get_stats(tsdf_volume* h, tsdf_stats* out, void* stream) {
    if (!h || !out) return TSDF_EINVAL;
    unsigned long long c[kCounterWords];
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(c, h->buf.counters, sizeof(c), hipMemcpyDeviceToHost, s) != hipSuccess) return TSDF_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TSDF_EHIP;
    const unsigned long long cap = (unsigned long long)h->cfg.pool_capacity;
    const unsigned long long used = c[kBlockCounter];
    std::memset(out, 0, sizeof(*out));
    out->pool_used = (int64_t)(used < cap ? used : cap);
    out->pool_overflow = (int64_t)(used > cap ? used - cap : 0);
    out->table_full = (int64_t)c[kTableFull];
    out->update_misses = (int64_t)c[kUpdateMisses];
    out->out_of_range = (int64_t)c[kOutOfRange];
    out->near_skipped = (int64_t)c[kNearSkipped];
    out->points_valid = (int64_t)c[kPointsValid];
    out->voxel_updates = (int64_t)c[kVoxelUpdates];
    out->walk_guard = (int64_t)c[kWalkGuard];
    out->probe_max = (int64_t)c[kProbeMax];
    for (int i = 0; i < kProbeBins; ++i) {
        out->probe_hist_alloc[i] = c[kHistAlloc + i];
        out->probe_hist_update[i] = c[kHistUpdate + i];
    }
    return TSDF_OK;
}

tsdf_status tsdf_export_blocks(tsdf_volume* h, int32_t* coords, float* tsdf, float* weight, float* r, float* g,
                               float* b, int64_t max_blocks, int64_t* n_blocks, void* stream) {
    if (!h || !n_blocks || max_blocks < 0) return TSDF_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned long long used = 0;
    const unsigned long long* dc = static_cast<const unsigned long long*>(h->buf.counters);
    if (hipMemcpyAsync(&used, dc + kBlockCounter, sizeof(used), hipMemcpyDeviceToHost, s) != hipSuccess)
        return TSDF_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TSDF_EHIP;
    const unsigned long long cap = (unsigned long long)h->cfg.pool_capacity;
    const int64_t n = (int64_t)(used < cap ? used : cap);
    *n_blocks = n;
    if (n > max_blocks) return TSDF_ESMALL;
    if (n == 0) return TSDF_OK;
    if (!coords) return TSDF_EINVAL;
    const unsigned long long entries = (unsigned long long)h->cfg.table_entries;
    hipLaunchKernelGGL(k_export_coords, dim3(grid_for(entries)), dim3(kThreads), 0, s,
                       static_cast<const Entry*>(h->buf.table), entries, (unsigned long long)n, coords);
    if (launched() != TSDF_OK) return TSDF_EHIP;
    const size_t bytes = (size_t)n * kBlockVoxels * sizeof(float);
    float* dst[5] = {tsdf, weight, r, g, b};
    const float* src[5] = {h->buf.tsdf, h->buf.weight, h->buf.r, h->buf.g, h->buf.b};
    for (int i = 0; i < 5; ++i)
        if (dst[i] && hipMemcpyAsync(dst[i], src[i], bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return TSDF_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TSDF_EHIP;
    return TSDF_OK;
}

void tsdf_destroy(tsdf_volume* h) { delete h; }

const char* tsdf_status_str(tsdf_status st) {
    switch (st) {
        case TSDF_OK: return "TSDF_OK";
        case TSDF_EINVAL: return "TSDF_EINVAL";
        case TSDF_EALIGN: return "TSDF_EALIGN";
        case TSDF_EHIP: return "TSDF_EHIP";
        case TSDF_ESMALL: return "TSDF_ESMALL";
    }
    return "TSDF_UNKNOWN";
}

}  // extern "C"
