// tsdf_capi.hip -- the C ABI of libtsdf_hip.so (include/tsdf.h): argument
// validation, the host-side volume handle, and kernel dispatch.  Memory is
// always the caller's ("What Irregularity Costs", section 3a: the harness
// allocates once and hands pointers through a C ABI).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "tsdf.h"
#include "tsdf_kernels.hpp"

using namespace tsdf;

namespace {

constexpr int kOwnerGridDefault = 2048;              // owner-update workgroups if the occupancy query fails
constexpr int64_t kDefaultFramePixels = 1 << 20;    // owner-mode record buffers, per call
constexpr int64_t kRunsPerPixel = 4;                // record capacity per pixel (a room frame needs ~2.7)
constexpr int64_t kSegmentsPerPixel = 2;            // (filing, block) segments per pixel: a room
                                                    //   frame needs ~0.15, coarse 160 x 120 ones ~0.9
constexpr int64_t kTilePixels = 256;                // an allocate workgroup's tile: it reserves in one
                                                    //   partition, which holds at least a tile's share

// Owner-mode scratch layout: per-frame counters, per-table-entry arrays,
// then the per-frame segment and record buffers (kParts partitions each).
struct ScratchLayout {
    size_t fc, desc, segs, recs, units, seg_list, blk_count, items, items_spill, seg_first_of, rescan, bytes;
    unsigned int item_part_cap, seg_part_cap, rec_part_cap;
};

ScratchLayout scratch_layout(int64_t entries, int64_t frame_pixels) {
    ScratchLayout L;
    const int64_t px = frame_pixels > 0 ? frame_pixels : kDefaultFramePixels;
    L.item_part_cap = (unsigned int)std::max<int64_t>(64, entries / (kParts / 2));
    const int64_t part_px = std::max<int64_t>((px + kParts - 1) / kParts, kTilePixels);
    L.seg_part_cap = (unsigned int)(kSegmentsPerPixel * part_px);
    L.rec_part_cap = (unsigned int)(kRunsPerPixel * part_px);
    size_t o = 0;
    L.fc = o;                         // 16-byte aligned pieces first
    o += 2 * sizeof(FrameCounters);
    L.desc = o;
    o += sizeof(ItemDesc) * (size_t)entries;
    L.segs = o;
    o += sizeof(Segment) * (size_t)kParts * L.seg_part_cap;
    L.recs = o;
    o += sizeof(RunRecord) * (size_t)kParts * L.rec_part_cap;
    L.units = o;                      // 8-byte pieces
    o += sizeof(uint2) * (size_t)kMaxUnits;
    L.seg_list = o;
    o += sizeof(uint2) * (size_t)kParts * L.seg_part_cap;
    L.blk_count = o;
    o += 8 * (size_t)entries;
    L.items = o;
    o += 4 * (size_t)kParts * L.item_part_cap;
    L.items_spill = o;
    o += 4 * (size_t)entries;
    L.seg_first_of = o;
    o += 4 * (size_t)entries;
    L.rescan = o;
    o += 4 * (size_t)entries;
    L.bytes = o;
    return L;
}

}  // namespace

namespace {

// Kernel timing: an event pair per launch, summed when read.
struct KernelClock {
    struct Span {
        int kernel;
        hipEvent_t start, end;
    };
    std::vector<Span> spans;
    std::vector<hipEvent_t> spare;
    bool failed = false;

    hipEvent_t take() {
        hipEvent_t e = nullptr;
        if (!spare.empty()) {
            e = spare.back();
            spare.pop_back();
        } else if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
        }
        return e;
    }
    void give(hipEvent_t e) {
        if (e) spare.push_back(e);
    }
    static void mark(void* ctx, int kernel, int phase, hipStream_t s) {
        KernelClock* c = static_cast<KernelClock*>(ctx);
        hipEvent_t e = c->take();
        if (!e || hipEventRecord(e, s) != hipSuccess) {
            c->give(e);
            c->failed = true;
            return;
        }
        if (phase == 0) {
            c->spans.push_back(Span{kernel, e, nullptr});
        } else if (!c->spans.empty() && c->spans.back().kernel == kernel && !c->spans.back().end) {
            c->spans.back().end = e;
        } else {
            c->give(e);
            c->failed = true;
        }
    }
    void drop() {
        for (Span& sp : spans) {
            give(sp.start);
            give(sp.end);
        }
        spans.clear();
    }
    ~KernelClock() {
        drop();
        for (hipEvent_t e : spare) (void)hipEventDestroy(e);
    }
};

}  // namespace

namespace {
constexpr int kMoreFrames = kMaxBatch - kArgFrames;   // frames of a call beyond the kernel arguments
constexpr size_t kCounterBytes = sizeof(unsigned long long) * kReplicas * kCounterWords;
static_assert(kCounterBytes % 16 == 0, "the frame table after the counters stays 16-byte aligned");
}  // namespace

// The scratch of tsdf_integrate_batch_noalloc: the owner update's per-call
// work lists (counters, segments, run records, per-slot run counts, item
// lists) for callers that cannot allocate.  One copy per GPU, held while the
// library is loaded.  Host code never uses this name as an address: its
// device address on each GPU comes from hipGetSymbolAddress (noalloc_base).
static __device__ __align__(256) unsigned char scratch[TSDF_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch_base[kMaxDevices];   // `scratch` on device d, once looked up

// The device address of `scratch` on device `dev` (looked up once per
// device, with that device current); nullptr if the lookup fails.
void* noalloc_base(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_lock);
    if (g_scratch_base[dev]) return g_scratch_base[dev];
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return nullptr;
    g_scratch_base[dev] = p;
    return p;
}
}  // namespace

struct tsdf_volume {
    tsdf_config cfg;
    tsdf_buffers buf;
    int device;                 // the GPU current at tsdf_create (where the buffers live)
    unsigned int mask;
    unsigned int serial;        // allocate calls so far (selects the per-call counter set)
    int owner_grid;             // owner-update workgroups: as many as the device holds at once
    bool pending;               // an owner-mode allocate whose update has not run yet
    int32_t n_last;             // the frames of that allocate
    tsdf_frame last[TSDF_MAX_BATCH];
    KernelClock* clock;         // non-null while kernel timing is on
    LaunchTimer timer;
};

namespace {

const LaunchTimer* timer_of(const tsdf_volume* h) { return h->clock ? &h->timer : nullptr; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t resolved_entries(const tsdf_config* c) {
    return c->table_entries ? c->table_entries : tsdf_table_entries_for(c->pool_capacity);
}

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
    a.probe_limit = h->cfg.probe_limit > 0 ? (unsigned int)h->cfg.probe_limit : 0xFFFFFFFFu;
    a.reproject = h->cfg.occlusion == TSDF_OCCLUSION_REPROJECT ? 1 : 0;
    return a;
}

// The owner update's work lists laid out in `scratch_base` for calls of up to
// `pixels` pixels (the volume's scratch: its configured max_batch_pixels).
OwnerArgs owner_args_at(const tsdf_volume* h, unsigned int serial, void* scratch_base, int64_t pixels) {
    OwnerArgs o;
    std::memset(&o, 0, sizeof(o));
    o.build_items = h->cfg.update_mode == TSDF_UPDATE_OWNER;
    o.parity = serial & 1u;
    if (!o.build_items) return o;
    const ScratchLayout L = scratch_layout(h->cfg.table_entries, pixels);
    char* base = static_cast<char*>(scratch_base);
    o.fc = reinterpret_cast<FrameCounters*>(base + L.fc);
    o.items = reinterpret_cast<unsigned int*>(base + L.items);
    o.items_spill = reinterpret_cast<unsigned int*>(base + L.items_spill);
    o.seg_first_of = reinterpret_cast<unsigned int*>(base + L.seg_first_of);
    o.blk_count = reinterpret_cast<unsigned long long*>(base + L.blk_count);
    o.rescan = reinterpret_cast<unsigned int*>(base + L.rescan);
    o.desc = reinterpret_cast<ItemDesc*>(base + L.desc);
    o.segs = reinterpret_cast<Segment*>(base + L.segs);
    o.recs = reinterpret_cast<RunRecord*>(base + L.recs);
    o.units = reinterpret_cast<uint2*>(base + L.units);
    o.unit_target = (unsigned int)std::min<int64_t>(kMaxUnits, 4 * (int64_t)std::max(1, h->owner_grid));
    o.seg_list = reinterpret_cast<uint2*>(base + L.seg_list);
    o.item_part_cap = L.item_part_cap;
    o.seg_part_cap = L.seg_part_cap;
    o.rec_part_cap = L.rec_part_cap;
    return o;
}

OwnerArgs owner_args(const tsdf_volume* h, unsigned int serial) {
    return owner_args_at(h, serial, h->buf.scratch, h->cfg.max_batch_pixels);
}

unsigned int next_serial(const tsdf_volume* h) { return h->serial + 1 == 0xFFFFFFFFu ? 1u : h->serial + 1; }

// init arguments: the owner-mode arrays that must start zeroed
bool init_volume(const tsdf_volume* h, bool whole_pool, hipStream_t s) {
    const OwnerArgs own = owner_args(h, 0);
    return launch_init(volume_args(h), (unsigned long long)h->cfg.table_entries, whole_pool,
                       own.build_items ? &own : nullptr, s);
}

// Validate a frame and fill the launch arguments.  *empty is set for a frame
// without pixels (nothing to launch).
tsdf_status frame_args(const tsdf_volume* h, const tsdf_frame* fr, bool need_rgb, FrameArgs* a, bool* empty) {
    if (!fr) return TSDF_EINVAL;
    if (fr->width < 0 || fr->height < 0 || fr->width > TSDF_MAX_FRAME_SIDE || fr->height > TSDF_MAX_FRAME_SIDE)
        return TSDF_EINVAL;
    const int64_t pixels = (int64_t)fr->width * fr->height;
    if (pixels > ((int64_t)1 << 31) - 1) return TSDF_EINVAL;
    *empty = pixels == 0;
    if (*empty) return TSDF_OK;
    if (!fr->depth || (need_rgb && !fr->rgb)) return TSDF_EINVAL;
    if (!std::isfinite(fr->fx) || !std::isfinite(fr->fy) || fr->fx == 0.0f || fr->fy == 0.0f) return TSDF_EINVAL;
    if (!std::isfinite(fr->cx) || !std::isfinite(fr->cy)) return TSDF_EINVAL;
    for (int i = 0; i < 9; ++i)
        if (!std::isfinite(fr->R[i])) return TSDF_EINVAL;
    for (int i = 0; i < 3; ++i)
        if (!std::isfinite(fr->t[i])) return TSDF_EINVAL;
    // R must be a rotation (to float precision): the update maps world
    // points back to pixels with its transpose
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double dot = 0.0;
            for (int k = 0; k < 3; ++k) dot += (double)fr->R[3 * i + k] * fr->R[3 * j + k];
            if (std::fabs(dot - (i == j ? 1.0 : 0.0)) > 1e-4) return TSDF_EINVAL;
        }
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
    a->tiles_x = (fr->width + 15) / 16;
    const int tiles_y = (fr->height + 15) / 16;
    a->n_tiles = a->tiles_x * tiles_y;
    a->tiles_per_xcd = (a->n_tiles + 7) / 8;
    return TSDF_OK;
}

bool same_frame(const tsdf_frame& a, const tsdf_frame& b) { return std::memcmp(&a, &b, sizeof(a)) == 0; }

// A call's frames: the first kArgFrames in the kernel arguments, the rest
// staged for the device table.
struct Batch {
    BatchArgs args;
    FrameArgs more[kMoreFrames];
};

// Validate n frames and gather the non-empty ones into a batch.
tsdf_status batch_args(const tsdf_volume* h, const tsdf_frame* frames, int32_t n, bool need_rgb, Batch* b) {
    if (!frames || n < 0 || n > TSDF_MAX_BATCH) return TSDF_EINVAL;
    BatchArgs& a = b->args;
    a.n = 0;
    a.tile_grid = 8;
    a.more = nullptr;
    for (int32_t i = 0; i < n; ++i) {
        FrameArgs fa;
        bool empty = false;
        const tsdf_status st = frame_args(h, frames + i, need_rgb, &fa, &empty);
        if (st != TSDF_OK) return st;
        if (empty) continue;
        if (a.n < kArgFrames)
            a.f[a.n] = fa;
        else
            b->more[a.n - kArgFrames] = fa;
        ++a.n;
        a.tile_grid = std::max(a.tile_grid, tile_grid(fa));
    }
    return TSDF_OK;
}

// Write the launch parameters of the frames beyond the kernel arguments to
// the device table (after the statistics in the counters buffer), ahead of
// the call's kernels on stream s: small kernels carry them in their own
// arguments, so nothing is allocated and no host memory must outlive the call.
tsdf_status stage_frames(tsdf_volume* h, Batch* b, hipStream_t s) {
    const int n_more = b->args.n - kArgFrames;
    if (n_more <= 0) return TSDF_OK;
    FrameArgs* table = reinterpret_cast<FrameArgs*>(static_cast<char*>(h->buf.counters) + kCounterBytes);
    if (!launch_store_frames(b->more, n_more, table, s)) return TSDF_EHIP;
    b->args.more = table;
    return TSDF_OK;
}

tsdf_status do_allocate(tsdf_volume* h, const BatchArgs& b, hipStream_t s) {
    if (h->pending && !launch_discard(volume_args(h), owner_args(h, h->serial), s, timer_of(h))) return TSDF_EHIP;
    h->pending = false;
    const unsigned int serial = next_serial(h);
    if (!launch_allocate(b, volume_args(h), owner_args(h, serial), s, timer_of(h))) return TSDF_EHIP;
    h->serial = serial;
    return TSDF_OK;
}

tsdf_status do_update(tsdf_volume* h, const BatchArgs& b, hipStream_t s) {
    if (h->cfg.update_mode == TSDF_UPDATE_RAYS)
        return launch_update_rays(b, volume_args(h), s, timer_of(h)) ? TSDF_OK : TSDF_EHIP;
    return launch_update_owner(b, volume_args(h), owner_args(h, h->serial), h->owner_grid, s, timer_of(h))
               ? TSDF_OK
               : TSDF_EHIP;
}

}  // namespace

extern "C" {

int64_t tsdf_table_entries_for(int64_t pool_capacity) {
    if (pool_capacity < 1 || pool_capacity > TSDF_MAX_POOL_BLOCKS) return -1;
    int64_t t = 1;
    while (t < 2 * pool_capacity) t <<= 1;
    return t;
}

size_t tsdf_counters_bytes(void) { return kCounterBytes + sizeof(FrameArgs) * kMoreFrames; }

size_t tsdf_scratch_bytes(const tsdf_config* config) {
    if (!config || config->update_mode != TSDF_UPDATE_OWNER) return 0;
    const int64_t entries = resolved_entries(config);
    if (entries <= 0 || config->max_batch_pixels < 0 || config->max_batch_pixels > ((int64_t)1 << 28)) return 0;
    return scratch_layout(entries, config->max_batch_pixels).bytes;
}

tsdf_status tsdf_create(const tsdf_config* config, const tsdf_buffers* buffers, void* stream, tsdf_volume** out) {
    if (!config || !buffers || !out) return TSDF_EINVAL;
    *out = nullptr;
    if (!finite_pos(config->voxel_size) || !finite_pos(config->trunc)) return TSDF_EINVAL;
    if (config->pool_capacity < 1 || config->pool_capacity > TSDF_MAX_POOL_BLOCKS) return TSDF_EINVAL;
    if (config->update_mode != TSDF_UPDATE_OWNER && config->update_mode != TSDF_UPDATE_RAYS) return TSDF_EINVAL;
    if (config->max_batch_pixels < 0 || config->max_batch_pixels > ((int64_t)1 << 28)) return TSDF_EINVAL;
    if (config->probe_limit < 0) return TSDF_EINVAL;
    if (config->occlusion != TSDF_OCCLUSION_RAY && config->occlusion != TSDF_OCCLUSION_REPROJECT) return TSDF_EINVAL;
    const int64_t entries = resolved_entries(config);
    if (!is_pow2(entries) || entries < 2 * config->pool_capacity || entries > TSDF_MAX_TABLE_ENTRIES)
        return TSDF_EINVAL;
    const tsdf_buffers& b = *buffers;
    if (!b.table || !b.tsdf || !b.weight || !b.r || !b.g || !b.b || !b.counters) return TSDF_EINVAL;
    if (config->update_mode == TSDF_UPDATE_OWNER && !b.scratch) return TSDF_EINVAL;
    if (!aligned16(b.table) || !aligned16(b.tsdf) || !aligned16(b.weight) || !aligned16(b.r) ||
        !aligned16(b.g) || !aligned16(b.b) || !aligned16(b.counters) || !aligned16(b.scratch))
        return TSDF_EALIGN;

    tsdf_volume* h = new (std::nothrow) tsdf_volume;
    if (!h) return TSDF_EINVAL;
    std::memset(h, 0, sizeof(*h));
    h->cfg = *config;
    h->cfg.table_entries = entries;
    h->buf = b;
    h->mask = (unsigned int)(entries - 1);
    if (hipGetDevice(&h->device) != hipSuccess) h->device = 0;
    (void)noalloc_base(h->device);   // the no-allocation entry point's scratch, looked up once per GPU
    h->owner_grid = owner_grid(config->occlusion == TSDF_OCCLUSION_REPROJECT);
    if (h->owner_grid <= 0) h->owner_grid = kOwnerGridDefault;
    if (!init_volume(h, true, static_cast<hipStream_t>(stream))) {
        delete h;
        return TSDF_EHIP;
    }
    *out = h;
    return TSDF_OK;
}

tsdf_status tsdf_reset(tsdf_volume* h, void* stream) {
    if (!h) return TSDF_EINVAL;
    h->pending = false;
    return init_volume(h, false, static_cast<hipStream_t>(stream)) ? TSDF_OK : TSDF_EHIP;
}

tsdf_status tsdf_allocate_batch(tsdf_volume* h, const tsdf_frame* frames, int32_t n_frames, void* stream) {
    if (!h) return TSDF_EINVAL;
    Batch b;
    const tsdf_status st = batch_args(h, frames, n_frames, false, &b);
    if (st != TSDF_OK || b.args.n == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const tsdf_status sf = stage_frames(h, &b, s);
    if (sf != TSDF_OK) return sf;
    const tsdf_status a = do_allocate(h, b.args, s);
    if (a == TSDF_OK && h->cfg.update_mode == TSDF_UPDATE_OWNER) {
        h->pending = true;
        h->n_last = n_frames;
        std::memcpy(h->last, frames, sizeof(tsdf_frame) * (size_t)n_frames);
    }
    return a;
}

tsdf_status tsdf_update_batch(tsdf_volume* h, const tsdf_frame* frames, int32_t n_frames, void* stream) {
    if (!h) return TSDF_EINVAL;
    Batch b;
    const tsdf_status st = batch_args(h, frames, n_frames, true, &b);
    if (st != TSDF_OK || b.args.n == 0) return st;
    if (h->cfg.update_mode == TSDF_UPDATE_OWNER) {
        if (!h->pending || h->n_last != n_frames) return TSDF_EINVAL;
        for (int32_t i = 0; i < n_frames; ++i)
            if (!same_frame(h->last[i], frames[i])) return TSDF_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const tsdf_status sf = stage_frames(h, &b, s);
    if (sf != TSDF_OK) return sf;
    if (h->cfg.update_mode == TSDF_UPDATE_OWNER) h->pending = false;
    return do_update(h, b.args, s);
}

tsdf_status tsdf_allocate(tsdf_volume* h, const tsdf_frame* frame, void* stream) {
    return tsdf_allocate_batch(h, frame, 1, stream);
}

tsdf_status tsdf_update(tsdf_volume* h, const tsdf_frame* frame, void* stream) {
    return tsdf_update_batch(h, frame, 1, stream);
}

tsdf_status tsdf_integrate_batch(tsdf_volume* h, const tsdf_frame* frames, int32_t n_frames, void* stream) {
    if (!h) return TSDF_EINVAL;
    Batch b;
    const tsdf_status st = batch_args(h, frames, n_frames, true, &b);
    if (st != TSDF_OK || b.args.n == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const tsdf_status sf = stage_frames(h, &b, s);
    if (sf != TSDF_OK) return sf;
    const tsdf_status a = do_allocate(h, b.args, s);
    if (a != TSDF_OK) return a;
    return do_update(h, b.args, s);
}

tsdf_status tsdf_integrate(tsdf_volume* h, const tsdf_frame* frame, void* stream) {
    return tsdf_integrate_batch(h, frame, 1, stream);
}

tsdf_status tsdf_integrate_batch_noalloc(tsdf_volume* h, const tsdf_frame* frames, int32_t n_frames, void* stream) {
    if (!h) return TSDF_EINVAL;
    Batch b;
    const tsdf_status st = batch_args(h, frames, n_frames, true, &b);
    if (st != TSDF_OK || b.args.n == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const VolumeArgs v = volume_args(h);
    if (h->cfg.update_mode == TSDF_UPDATE_RAYS) {            // no work lists: nothing to place
        if (stage_frames(h, &b, s) != TSDF_OK) return TSDF_EHIP;
        const unsigned int serial = next_serial(h);
        if (!launch_allocate(b.args, v, owner_args(h, serial), s, nullptr)) return TSDF_EHIP;
        h->serial = serial;
        return launch_update_rays(b.args, v, s, nullptr) ? TSDF_OK : TSDF_EHIP;
    }
    int64_t pixels = 0;
    for (int32_t i = 0; i < n_frames; ++i) pixels += (int64_t)frames[i].width * frames[i].height;
    // (the layout's per-partition capacities are 32-bit: size them only for
    // pixel counts a configuration may state)
    if (pixels > ((int64_t)1 << 28) ||
        scratch_layout(h->cfg.table_entries, pixels).bytes > TSDF_NOALLOC_SCRATCH_BYTES)
        return TSDF_ELIMIT;
    void* base = noalloc_base(h->device);
    if (!base) return TSDF_EHIP;
    if (stage_frames(h, &b, s) != TSDF_OK) return TSDF_EHIP;
    // an allocate still waiting for its update is dropped, as by any allocate
    if (h->pending && !launch_discard(v, owner_args(h, h->serial), s, nullptr)) return TSDF_EHIP;
    h->pending = false;
    const unsigned int serial = next_serial(h);
    const OwnerArgs own = owner_args_at(h, serial, base, pixels);
    if (!launch_fresh_call(v, own, (unsigned long long)h->cfg.table_entries, s)) return TSDF_EHIP;
    if (!launch_allocate(b.args, v, own, s, nullptr)) return TSDF_EHIP;
    if (!launch_update_owner(b.args, v, own, h->owner_grid, s, nullptr)) return TSDF_EHIP;
    // the volume's own work lists: ready for its next call, whose fresh
    // blocks start after this call's
    h->serial = serial;
    const OwnerArgs mine = owner_args(h, next_serial(h));
    return launch_hand_back(v, mine.fc + mine.parity, s) ? TSDF_OK : TSDF_EHIP;
}

tsdf_status tsdf_get_stats(tsdf_volume* h, tsdf_stats* out, void* stream) {
    if (!h || !out) return TSDF_EINVAL;
    static thread_local unsigned long long c[kReplicas * kCounterWords];
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(c, h->buf.counters, sizeof(c), hipMemcpyDeviceToHost, s) != hipSuccess) return TSDF_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TSDF_EHIP;
    unsigned long long sum[kCounterWords] = {0};
    for (int r = 0; r < kReplicas; ++r)
        for (int k = 0; k < kCounterWords; ++k) {
            const unsigned long long v = c[r * kCounterWords + k];
            sum[k] = k == kProbeMax ? std::max(sum[k], v) : sum[k] + v;
        }
    const unsigned long long cap = (unsigned long long)h->cfg.pool_capacity;
    const unsigned long long used = c[kBlockCounter];          // copy 0 holds the pool-index counter
    std::memset(out, 0, sizeof(*out));
    out->pool_used = (int64_t)(used < cap ? used : cap);
    out->pool_overflow = (int64_t)(used > cap ? used - cap : 0);
    out->table_full = (int64_t)sum[kTableFull];
    out->update_misses = (int64_t)sum[kUpdateMisses];
    out->out_of_range = (int64_t)sum[kOutOfRange];
    out->near_skipped = (int64_t)sum[kNearSkipped];
    out->points_valid = (int64_t)sum[kPointsValid];
    out->voxel_updates = (int64_t)sum[kVoxelUpdates];
    out->walk_guard = (int64_t)sum[kWalkGuard];
    out->probe_max = (int64_t)sum[kProbeMax];
    out->fallback_blocks = (int64_t)sum[kFallbackBlocks];
    out->probe_exhausted = (int64_t)sum[kProbeExhausted];
    for (int i = 0; i < kProbeBins; ++i) {
        out->probe_hist_alloc[i] = sum[kHistAlloc + i];
        out->probe_hist_update[i] = sum[kHistUpdate + i];
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
    if (!launch_export_coords(volume_args(h), (unsigned long long)h->cfg.table_entries, (unsigned long long)n,
                              coords, s))
        return TSDF_EHIP;
    const size_t bytes = (size_t)n * kBlockVoxels * sizeof(float);
    float* dst[5] = {tsdf, weight, r, g, b};
    const float* src[5] = {h->buf.tsdf, h->buf.weight, h->buf.r, h->buf.g, h->buf.b};
    for (int i = 0; i < 5; ++i)
        if (dst[i] && hipMemcpyAsync(dst[i], src[i], bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return TSDF_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TSDF_EHIP;
    return TSDF_OK;
}

tsdf_status tsdf_extract_mesh(tsdf_volume* h, float* positions, int32_t* keys, int64_t max_triangles,
                              int64_t* n_triangles, void* stream) {
    if (!h || !n_triangles || max_triangles < 0 || (max_triangles > 0 && !positions)) return TSDF_EINVAL;
    if ((uintptr_t)positions % 4 != 0 || (uintptr_t)keys % 4 != 0) return TSDF_EALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned long long* counter = static_cast<unsigned long long*>(h->buf.counters) + kMeshTriangles;
    if (!launch_mesh(volume_args(h), (unsigned long long)h->cfg.table_entries, counter, positions,
                     reinterpret_cast<int*>(keys), (unsigned long long)max_triangles, s))
        return TSDF_EHIP;
    unsigned long long n = 0;
    if (hipMemcpyAsync(&n, counter, sizeof(n), hipMemcpyDeviceToHost, s) != hipSuccess) return TSDF_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TSDF_EHIP;
    *n_triangles = (int64_t)n;
    return (int64_t)n > max_triangles ? TSDF_ESMALL : TSDF_OK;
}

tsdf_status tsdf_set_kernel_timing(tsdf_volume* h, int32_t enable) {
    if (!h) return TSDF_EINVAL;
    if (enable && !h->clock) {
        h->clock = new (std::nothrow) KernelClock;
        if (!h->clock) return TSDF_EINVAL;
        h->timer.ctx = h->clock;
        h->timer.mark = &KernelClock::mark;
    } else if (!enable && h->clock) {
        delete h->clock;
        h->clock = nullptr;
    }
    return TSDF_OK;
}

tsdf_status tsdf_kernel_times(tsdf_volume* h, tsdf_kernel_time* out, int32_t max_entries, int32_t* n_entries) {
    if (!h || !n_entries || max_entries < 0 || (max_entries > 0 && !out)) return TSDF_EINVAL;
    *n_entries = 0;
    if (!h->clock) return TSDF_EINVAL;
    KernelClock& c = *h->clock;
    int64_t launches[kKernelIds] = {0};
    double ms[kKernelIds] = {0.0};
    bool ok = !c.failed;
    for (const KernelClock::Span& sp : c.spans) {
        float t = 0.0f;
        if (!sp.end || hipEventSynchronize(sp.end) != hipSuccess ||
            hipEventElapsedTime(&t, sp.start, sp.end) != hipSuccess) {
            ok = false;
            continue;
        }
        ++launches[sp.kernel];
        ms[sp.kernel] += t;
    }
    c.drop();
    c.failed = false;
    if (!ok) return TSDF_EHIP;
    int32_t n = 0;
    for (int k = 0; k < kKernelIds; ++k) {
        if (!launches[k]) continue;
        if (n < max_entries) {
            tsdf_kernel_time& e = out[n];
            std::memset(&e, 0, sizeof(e));
            std::snprintf(e.name, sizeof(e.name), "%s", kernel_name(k));
            e.launches = launches[k];
            e.total_ms = ms[k];
        }
        ++n;
    }
    *n_entries = n;
    return n > max_entries ? TSDF_ESMALL : TSDF_OK;
}

void tsdf_destroy(tsdf_volume* h) {
    if (!h) return;
    delete h->clock;
    delete h;
}

const char* tsdf_status_str(tsdf_status st) {
    switch (st) {
        case TSDF_OK: return "TSDF_OK";
        case TSDF_EINVAL: return "TSDF_EINVAL";
        case TSDF_EALIGN: return "TSDF_EALIGN";
        case TSDF_EHIP: return "TSDF_EHIP";
        case TSDF_ESMALL: return "TSDF_ESMALL";
        case TSDF_ELIMIT: return "TSDF_ELIMIT";
    }
    return "TSDF_UNKNOWN";
}

}  // extern "C"
