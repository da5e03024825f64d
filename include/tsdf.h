/*
 * tsdf.h -- C ABI of libtsdf_hip.so, the MI355X (gfx950) implementation of
 * the integrate path of hash-blocked TSDF fusion.
 *
 * The method is the one in "What Irregularity Costs: CUDA C++, Rust, and
 * Triton on a Hash-Blocked GPU Workload" (section 3): voxels are grouped in
 * blocks of 8^3 = 512; an open-addressed, linear-probing hash table of
 * 16-byte entries (64-bit packed key, 32-bit block index, 4 bytes padding)
 * maps block coordinates to indices in a flat pool of five parallel float
 * arrays (TSDF sum, weight, R, G, B sums); integration is two kernels over
 * the same points, `allocate` (walk the band, insert missing blocks with one
 * 64-bit compare-exchange per key) and `update` (look blocks up, five atomic
 * additions per voxel, storing sums rather than means).  As in the paper's
 * section 3a harness, all memory is allocated by the caller and handed over
 * as plain pointers; the library never allocates, frees or reshapes it.
 *
 * Conventions for every entry point:
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call that launches work enqueues it on `stream` and returns without
 *     waiting, except tsdf_export_blocks and tsdf_get_stats, which wait.
 *   - Invalid arguments return a negative status synchronously and enqueue
 *     nothing.  A failed HIP launch or copy returns TSDF_EHIP.
 *   - Data loss is never a status code: pool exhaustion, a full table and
 *     misses are counters read back by tsdf_get_stats (the paper's
 *     section 3a requires pool-exhaustion reporting, section 7 shows why
 *     probe exhaustion must be reported too).  No block is ever dropped
 *     without being counted.
 *   - A volume is used from one stream at a time; calls on one volume must
 *     not overlap.  Frame memory must stay valid until the enqueued work
 *     has run.
 */
#ifndef TSDF_H
#define TSDF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TSDF_OK = 0,
    TSDF_EINVAL = -1,   /* invalid argument: null pointer, bad size or parameter */
    TSDF_EALIGN = -2,   /* a buffer is not 16-byte aligned */
    TSDF_EHIP = -3,     /* a HIP launch or copy failed */
    TSDF_ESMALL = -4,   /* the caller's output buffers are too small */
    TSDF_ELIMIT = -5    /* the call needs more than tsdf_integrate_batch_noalloc's fixed scratch */
} tsdf_status;

/* Largest pool, in blocks; the pool index of a block must fit 32 bits with
 * two sentinel values left over. */
#define TSDF_MAX_POOL_BLOCKS (1LL << 30)
/* Largest table, in entries. */
#define TSDF_MAX_TABLE_ENTRIES (1LL << 31)
/* Largest number of cells one point's band walk may visit (a frame whose
 * intrinsics allow more is rejected with TSDF_EINVAL). */
#define TSDF_MAX_WALK 4096
/* Most frames one tsdf_integrate_batch call takes. */
#define TSDF_MAX_BATCH 128
/* Largest frame width and height, in pixels (a pixel position is recorded
 * as two 16-bit halves). */
#define TSDF_MAX_FRAME_SIDE 65535
/* Bins of the probe-depth histograms: bin i counts probes of i+1 slots,
 * the last bin counts TSDF_PROBE_BINS slots or more. */
#define TSDF_PROBE_BINS 32

typedef struct tsdf_volume tsdf_volume;     /* opaque host-side handle */

/* How tsdf_update adds a frame's contributions (both give the same sums):
 *   TSDF_UPDATE_OWNER  each block the frame touched is handed to one
 *                      workgroup, which replays the band walks that reach it,
 *                      sums them in LDS and read-modify-writes the block's
 *                      voxels with plain coalesced loads and stores (a block
 *                      whose runs overflow the scratch record buffers is
 *                      rescanned from the pixels its band can be seen through);
 *   TSDF_UPDATE_RAYS   one thread per point walks its band, looks each block
 *                      run up and adds with five f32 atomics per voxel (the
 *                      paper's section 3 shape). */
typedef enum { TSDF_UPDATE_OWNER = 0, TSDF_UPDATE_RAYS = 1 } tsdf_update_mode;

/* The occlusion test both passes apply to every voxel a band walk visits
 * (section 3 of the paper: allocate and update apply the same test; the
 * pages do not define it).  Both readings keep a voxel only inside the band,
 * |d - zc| <= trunc, where d is the point's depth and zc the camera depth of
 * the voxel centre:
 *   TSDF_OCCLUSION_RAY        nothing more: a centre more than trunc behind
 *                             the point's own depth is hidden (the band's far
 *                             end), evaluable from the point alone (default);
 *   TSDF_OCCLUSION_REPROJECT  also hidden when the depth image shows a
 *                             surface more than trunc in front of the centre
 *                             at the pixel nearest to the centre's projection
 *                             (no valid depth there, or a projection outside
 *                             the image or behind the camera: not hidden). */
typedef enum { TSDF_OCCLUSION_RAY = 0, TSDF_OCCLUSION_REPROJECT = 1 } tsdf_occlusion;

typedef struct {
    float voxel_size;       /* metres, finite, > 0 */
    float trunc;            /* truncation distance, metres, finite, > 0 */
    int64_t pool_capacity;  /* blocks, 1 .. TSDF_MAX_POOL_BLOCKS */
    int64_t table_entries;  /* 0: tsdf_table_entries_for(pool_capacity); otherwise a power of
                               two >= 2 * pool_capacity (so the table is at most half full)
                               and <= TSDF_MAX_TABLE_ENTRIES */
    int32_t update_mode;    /* tsdf_update_mode */
    int64_t max_batch_pixels; /* owner mode: total pixels of the frames one call integrates,
                               which sizes the run-record buffers (0: 2^20); larger calls
                               still integrate exactly, but blocks whose records do not fit
                               are rescanned pixel by pixel (slower) */
    int32_t probe_limit;    /* 0: probes run until they find the key or a free slot (the
                               paper's CUDA C++ and Rust probes, section 7).  n > 0: a
                               negative control reproducing the bounded probe of the
                               paper's Triton arm (section 7): a table operation gives up
                               after n slots; such keys are counted in probe_exhausted and
                               their contributions in update_misses.  Not for production. */
    int32_t occlusion;      /* tsdf_occlusion (zero-initialised configs get TSDF_OCCLUSION_RAY) */
} tsdf_config;

/* Device memory owned by the caller, all 16-byte aligned. */
typedef struct {
    void* table;            /* table_entries * 16 bytes; entry = {uint64 key, uint32 pool index,
                               uint32 padding} */
    float* tsdf;            /* pool_capacity * 512 floats each: per-voxel sums of the */
    float* weight;          /*   normalised signed distance (sdf / trunc), of the weight, */
    float* r;               /*   and of the colour channels (0..1).  Voxel v of block i is */
    float* g;               /*   element i * 512 + v, v = x + 8 y + 64 z within the block. */
    float* b;               /* The library relies on pool blocks it has not handed out
                               holding zeros (tsdf_create and tsdf_reset clear them): a
                               block's first sums are written without reading it. */
    void* counters;         /* tsdf_counters_bytes() bytes: statistics, then the launch
                               parameters of a batch's frames beyond the 32nd */
    void* scratch;          /* tsdf_scratch_bytes(config) bytes (the owner update's work
                               list); may be NULL when that is 0 */
} tsdf_buffers;

/* One depth frame.  Pointers are device memory. */
typedef struct {
    const float* depth;     /* height * width floats, row-major, metres of camera z;
                               0, negative or non-finite = no measurement */
    const uint8_t* rgb;     /* height * width * 3 bytes, row-major, R G B interleaved;
                               needed by update and integrate, ignored by allocate */
    int32_t width, height;  /* 0 .. TSDF_MAX_FRAME_SIDE; an empty frame is a no-op */
    float fx, fy, cx, cy;   /* pinhole intrinsics, pixels; pixel (u, v) looks along
                               ((u - cx) / fx, (v - cy) / fy, 1) in camera coordinates */
    float R[9];             /* camera-to-world rotation, row-major; must be orthonormal to
                               within 1e-4 (else TSDF_EINVAL) */
    float t[3];             /* camera position in the world, metres */
} tsdf_frame;

/* Counters accumulated since tsdf_create / tsdf_reset.  Point and voxel
 * counts are taken by tsdf_allocate (every call counts its frame). */
typedef struct {
    int64_t pool_used;       /* blocks holding a pool index (<= pool_capacity) */
    int64_t pool_overflow;   /* distinct keys inserted after the pool was full */
    int64_t table_full;      /* insertions that probed every table slot without room */
    int64_t update_misses;   /* kept voxel contributions lost: block without a pool index,
                                or key not inserted (full table, or probe_limit reached) */
    int64_t out_of_range;    /* points whose band leaves +-2^23 voxels */
    int64_t near_skipped;    /* points with 0 < depth <= trunc */
    int64_t points_valid;    /* points whose band was walked */
    int64_t voxel_updates;   /* kept (point, voxel) pairs */
    int64_t walk_guard;      /* walks cut at TSDF_MAX_WALK (never expected: always 0) */
    int64_t probe_max;       /* longest probe sequence seen, slots */
    int64_t fallback_blocks; /* owner update: blocks rescanned pixel by pixel because their
                                run records did not fit the scratch buffer (slower, exact) */
    int64_t probe_exhausted; /* table operations that gave up at probe_limit slots (0
                                unless the config sets a limit) */
    uint64_t probe_hist_alloc[TSDF_PROBE_BINS];   /* allocate: slots per table operation */
    uint64_t probe_hist_update[TSDF_PROBE_BINS];  /* ray-parallel update: slots per lookup */
} tsdf_stats;

/* Default table size for a pool: the smallest power of two >= 2 * pool_capacity
 * (section 3 of the paper: at most half full).  Returns -1 for an invalid capacity. */
int64_t tsdf_table_entries_for(int64_t pool_capacity);

/* Size of the counters buffer (the statistics, and a device table of the
 * launch parameters of up to TSDF_MAX_BATCH - 32 frames). */
size_t tsdf_counters_bytes(void);

/* Size of the scratch buffer a configuration needs (0 for TSDF_UPDATE_RAYS):
 * about 60 bytes per table entry plus 96 bytes per pixel of max_batch_pixels
 * (run records and their grouping by block; at least 16,384 pixels' worth).
 * 0 for a NULL or invalid config. */
size_t tsdf_scratch_bytes(const tsdf_config* config);

/* Validate the configuration and buffers, then enqueue the initialisation of
 * the volume on `stream`: every table entry empty (all bits set), counters
 * zero, the whole pool zero.  On success *out receives a new handle. */
tsdf_status tsdf_create(const tsdf_config* config, const tsdf_buffers* buffers, void* stream,
                        tsdf_volume** out);

/* Enqueue a reset to the state tsdf_create leaves: the used part of the pool
 * is zeroed, the table emptied and the counters cleared. */
tsdf_status tsdf_reset(tsdf_volume* volume, void* stream);

/* The allocate kernel (paper, section 3): for every point, walk its
 * truncation band; for each kept voxel make sure its block is in the table,
 * inserting it with a single 64-bit compare-exchange of the packed key and
 * taking the next pool index.  Block keys are de-duplicated within each
 * wavefront before probing.  The probe has no fixed bound: it stops at the
 * key, at an empty slot it wins, or after trying every slot (table_full).  A
 * key inserted after the pool is full gets no index (pool_overflow).  In
 * owner mode it also records, once per block, the blocks this frame touches
 * for the following tsdf_update. */
tsdf_status tsdf_allocate(tsdf_volume* volume, const tsdf_frame* frame, void* stream);

/* The update kernel (paper, section 3): the same walk and occlusion test;
 * each kept voxel receives sdf/trunc, 1, R/255, G/255, B/255 in the five
 * pool arrays (sums, not means).  Contributions to blocks without an index
 * count as update_misses.  Call after tsdf_allocate of the same frame
 * (stream order is the only ordering needed); in owner mode the call must
 * directly follow tsdf_allocate of an identical tsdf_frame, else
 * TSDF_EINVAL. */
tsdf_status tsdf_update(tsdf_volume* volume, const tsdf_frame* frame, void* stream);

/* tsdf_allocate then tsdf_update of one frame. */
tsdf_status tsdf_integrate(tsdf_volume* volume, const tsdf_frame* frame, void* stream);

/* Integrate n_frames (0 .. TSDF_MAX_BATCH) frames with one allocate launch
 * over all of them followed by one update: the result equals integrating
 * them one by one (the block set is the union, sums commute; which keys an
 * exhausted pool refuses may differ, their number does not), but each block
 * the batch touches is read and written once.  Frames may differ in size.
 * The launch parameters of frames beyond the 32nd are written to the device
 * table in the counters buffer by small kernels on the stream that carry
 * them in their arguments (the library allocates nothing for them). */
tsdf_status tsdf_integrate_batch(tsdf_volume* volume, const tsdf_frame* frames, int32_t n_frames, void* stream);

/* tsdf_integrate_batch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it): the same kernels and the same result, but the owner update's per-call
 * work lists live in a fixed scratch array inside the library, of
 * TSDF_NOALLOC_SCRATCH_BYTES per GPU (held from the moment the library is
 * loaded until the process ends), instead of the volume's scratch buffer.
 * The call allocates nothing: no device, pinned or event memory, and no
 * kernel timing (tsdf_set_kernel_timing does not cover it).
 * Limit (TSDF_ELIMIT, nothing enqueued): in owner mode the work lists of the
 * call must fit the array: tsdf_scratch_bytes of the volume's config with
 * max_batch_pixels set to the call's total pixels, i.e. about 60 bytes per
 * table entry plus 96 per pixel, at most TSDF_NOALLOC_SCRATCH_BYTES.
 * Ray-parallel volumes need no work lists.  Up to TSDF_MAX_BATCH frames.
 * Every call on one GPU shares that GPU's array, which keeps the previous
 * call's contents (each call clears what it needs): calls that overlap in
 * time on one GPU, on any volume or stream, race and must not be issued.
 * Mixing it with the other entry points on one volume is allowed: the
 * volume's own scratch is left ready for its next call. */
#define TSDF_NOALLOC_SCRATCH_BYTES (64u << 20)
tsdf_status tsdf_integrate_batch_noalloc(tsdf_volume* volume, const tsdf_frame* frames, int32_t n_frames,
                                         void* stream);

/* The two halves of tsdf_integrate_batch.  In owner mode tsdf_update_batch
 * must directly follow tsdf_allocate_batch of identical frames, else
 * TSDF_EINVAL; tsdf_allocate and tsdf_update are these with one frame. */
tsdf_status tsdf_allocate_batch(tsdf_volume* volume, const tsdf_frame* frames, int32_t n_frames, void* stream);
tsdf_status tsdf_update_batch(tsdf_volume* volume, const tsdf_frame* frames, int32_t n_frames, void* stream);

/* Copy every block holding a pool index to caller device memory, in pool
 * index order: coords (n x 3 int32 block coordinates) and, for each non-null
 * array pointer, n * 512 floats of that pool array.  *n_blocks receives n
 * (host memory).  Returns TSDF_ESMALL, copying nothing, if n > max_blocks.
 * Waits for the stream. */
tsdf_status tsdf_export_blocks(tsdf_volume* volume, int32_t* coords, float* tsdf, float* weight,
                               float* r, float* g, float* b, int64_t max_blocks, int64_t* n_blocks,
                               void* stream);

/* Surface extraction by marching tetrahedra (the paper extracts the surface
 * once, after integration, by marching tetrahedra: section 3; its gates
 * compare extracted surfaces: section 3a).  Samples are the voxel centres;
 * a voxel is observed iff its weight sum is > 0, inside iff its TSDF sum is
 * < 0, its value is the mean TSDF.  The cell between voxels k and k + (1,1,1)
 * is cut into six tetrahedra along that diagonal (for each ordering a, b, c
 * of the axes -- xyz, xzy, yxz, yzx, zxy, zyx -- the corners k, k + e_a,
 * k + e_a + e_b, k + (1,1,1)); tetrahedra with an unobserved corner are
 * skipped; each edge between an inside and an outside corner, from lattice
 * point p to p + d (d in {0,1}^3), holds one vertex at p + t d in voxel
 * units, t = v_p / (v_p - v_{p+d}), position ((p + t d) + 1/2) vs metres.
 * Triangles face from inside to outside.  Output, caller device memory:
 * positions (9 floats per triangle: x, y, z of its three vertices, metres)
 * and, if keys is not NULL, the vertices' names (12 int32 per triangle:
 * p_x, p_y, p_z, d_x | d_y << 1 | d_z << 2 per vertex; a vertex shared by
 * several triangles has the same name in each, so the soup can be welded).
 * *n_triangles (host) receives the number of triangles; only the first
 * max_triangles are written, and TSDF_ESMALL is returned if there are more.
 * Triangles come in no particular order.  Reads the volume; writes nothing
 * of it but a word of its counters buffer (not a statistic).  Waits for the
 * stream. */
tsdf_status tsdf_extract_mesh(tsdf_volume* volume, float* positions, int32_t* keys, int64_t max_triangles,
                              int64_t* n_triangles, void* stream);

/* Read the counters into *stats (host memory).  Waits for the stream. */
tsdf_status tsdf_get_stats(tsdf_volume* volume, tsdf_stats* stats, void* stream);

/* Per-kernel timing, for measurement (the paper's section 4 times each
 * stage on its own).  While enabled, every kernel the volume launches is
 * bracketed by two HIP events recorded on its launch stream.
 * tsdf_kernel_times waits for the events recorded so far, and writes one
 * entry per kernel that ran since timing was enabled or last read: its
 * name, launches and summed event-to-event milliseconds; then it clears the
 * sums.  *n_entries receives the number of entries (host memory); at most
 * max_entries are written, TSDF_ESMALL if more exist.  Disabling drops
 * unread records.  Timing costs two event records per launch. */
typedef struct {
    char name[32];          /* kernel name, e.g. "k_update_owner" */
    int64_t launches;
    double total_ms;
} tsdf_kernel_time;

tsdf_status tsdf_set_kernel_timing(tsdf_volume* volume, int32_t enable);
tsdf_status tsdf_kernel_times(tsdf_volume* volume, tsdf_kernel_time* out, int32_t max_entries,
                              int32_t* n_entries);

/* Free the handle (and its timing events).  Never frees caller memory. */
void tsdf_destroy(tsdf_volume* volume);

/* Name of a status code. */
const char* tsdf_status_str(tsdf_status status);

#ifdef __cplusplus
}
#endif

#endif /* TSDF_H */
