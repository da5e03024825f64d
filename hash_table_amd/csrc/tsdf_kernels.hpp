// tsdf_kernels.hpp -- host launch wrappers of the gfx950 kernels in
// tsdf_kernels.hip.  Each enqueues on `s` and returns false if the launch
// failed.
#pragma once

#include <hip/hip_runtime.h>

#include "tsdf_device.hpp"

namespace tsdf {

// Kernels, as the optional launch timer sees them.
enum KernelId {
    kKAllocate = 0,
    kKPlaceItems,
    kKPlaceSegments,
    kKUpdateOwner,
    kKUpdateRescan,
    kKDiscardItems,
    kKUpdateRays,
    kKernelIds
};
const char* kernel_name(int id);

// Called right before (phase 0) and after (phase 1) every launch of the
// integrate path when the caller passes one.
struct LaunchTimer {
    void* ctx;
    void (*mark)(void* ctx, int kernel, int phase, hipStream_t s);
};

// workgroups of the per-point kernels for a frame (a multiple of 8)
int tile_grid(const FrameArgs& f);

bool launch_allocate(const BatchArgs& b, const VolumeArgs& v, const OwnerArgs& o, hipStream_t s,
                     const LaunchTimer* t);
// group the batch's run records by block, then update every touched block
// (`grid` workgroups; owner_grid(reproject) is the number of the matching
// instantiation the device holds at once)
bool launch_update_owner(const BatchArgs& b, const VolumeArgs& v, const OwnerArgs& o, int grid, hipStream_t s,
                         const LaunchTimer* t);
int owner_grid(bool reproject);
// forget an allocate's records (no update followed it)
bool launch_discard(const VolumeArgs& v, const OwnerArgs& o, hipStream_t s, const LaunchTimer* t);
bool launch_update_rays(const BatchArgs& b, const VolumeArgs& v, hipStream_t s, const LaunchTimer* t);
// zero the pool (whole, or the used part), empty the table, clear the counters
// and (owner mode) the per-slot run counts and per-frame counters
bool launch_init(const VolumeArgs& v, unsigned long long table_entries, bool whole_pool, const OwnerArgs* own,
                 hipStream_t s);
// write the launch parameters of n frames into the device frame table, in
// stream order (small kernels carrying them in their arguments)
bool launch_store_frames(const FrameArgs* frames, int n, FrameArgs* table, hipStream_t s);
// a call whose owner-mode work lists live in memory other than the volume's
// scratch: clear its two per-call counter sets and per-slot run counts, and
// set its fresh-block start to the block counter's value before the call
bool launch_fresh_call(const VolumeArgs& v, const OwnerArgs& o, unsigned long long table_entries, hipStream_t s);
// after such a call: leave the volume's own counter set `next` (the one the
// volume's next call will use) as a call of its own would have
bool launch_hand_back(const VolumeArgs& v, FrameCounters* next, hipStream_t s);
// surface extraction (tsdf_mesh.hip): clears *counter, then counts every
// triangle in it and writes those below max_triangles (key may be null)
bool launch_mesh(const VolumeArgs& v, unsigned long long table_entries, unsigned long long* counter, float* pos,
                 int* key, unsigned long long max_triangles, hipStream_t s);
bool launch_export_coords(const VolumeArgs& v, unsigned long long table_entries, unsigned long long n_blocks,
                          int* coords, hipStream_t s);

}  // namespace tsdf
