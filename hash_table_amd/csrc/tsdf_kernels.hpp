// tsdf_kernels.hpp -- host launch wrappers of the gfx950 kernels in
// tsdf_kernels.hip.  Each enqueues on `s` and returns false if the launch
// failed.
#pragma once

#include <hip/hip_runtime.h>

#include "tsdf_device.hpp"

namespace tsdf {

// workgroups of the per-point kernels for a frame (a multiple of 8)
int tile_grid(const FrameArgs& f);

bool launch_allocate(const BatchArgs& b, const VolumeArgs& v, const OwnerArgs& o, hipStream_t s);
// group the batch's run records by block, then update every touched block
bool launch_update_owner(const BatchArgs& b, const VolumeArgs& v, const OwnerArgs& o, int grid, hipStream_t s);
// forget an allocate's records (no update followed it)
bool launch_discard(const VolumeArgs& v, const OwnerArgs& o, hipStream_t s);
bool launch_update_rays(const BatchArgs& b, const VolumeArgs& v, hipStream_t s);
// zero the pool (whole, or the used part), empty the table, clear the counters
// and (owner mode) the per-slot run counts and per-frame counters
bool launch_init(const VolumeArgs& v, unsigned long long table_entries, bool whole_pool, const OwnerArgs* own,
                 hipStream_t s);
bool launch_export_coords(const VolumeArgs& v, unsigned long long table_entries, unsigned long long n_blocks,
                          int* coords, hipStream_t s);

}  // namespace tsdf
