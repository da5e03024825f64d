// tsdf_device.hpp -- device-side pieces of the integrate path for gfx950:
// the band walk of one depth point, the packed block key, its hash, and the
// hash-table probe loops.  Method: "What Irregularity Costs: CUDA C++, Rust,
// and Triton on a Hash-Blocked GPU Workload", section 3 (blocks of 8^3
// voxels, 16-byte entries with a 64-bit key packing three axes biased by
// 2^20 into 21 bits, linear probing, insertion by a single compare-exchange
// of the key, pool of five float arrays holding sums).
//
// Float rules of the walk (shared by construction with the checking
// implementation, written separately there): IEEE f32, round to nearest, no
// FMA contraction (built with -ffp-contract=off), correctly rounded division,
// every expression evaluated in the order written below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsdf {

constexpr unsigned long long kEmptyKey = ~0ull;     // table initialised to all ones
constexpr unsigned int kUnpublished = 0xFFFFFFFFu;  // index not yet stored
constexpr unsigned int kNoIndex = 0xFFFFFFFEu;      // key inserted after the pool filled
constexpr int kKeyBias = 1 << 20;                   // per-axis bias of the packed key
constexpr float kRangeLimit = 8388600.0f;           // |voxel coord| limit: 2^23 - 8
constexpr float kStillAxis = 1e-30f;                // |direction| at or below: axis never steps
constexpr int kBlockVoxels = 512;
constexpr int kProbeBins = 32;

// Counter words (uint64) of one replica of the caller's counters buffer.
// Statistics are spread over kReplicas copies (workgroup w adds to copy
// w mod kReplicas) because same-address atomics serialise; readers sum the
// copies.  The pool-index counter lives in copy 0 only.
enum CounterWord {
    kBlockCounter = 0,   // next pool index; may run past the capacity (copy 0 only)
    kTableFull,
    kUpdateMisses,
    kOutOfRange,
    kNearSkipped,
    kPointsValid,
    kVoxelUpdates,
    kWalkGuard,
    kProbeMax,
    kFallbackBlocks,     // owner update: blocks rescanned because their runs did not fit
    kProbeExhausted,     // table operations that stopped at the configured probe limit
    kMeshTriangles,      // triangles of the last surface extraction (copy 0 only; not a statistic)
    kHistAlloc = 16,
    kHistUpdate = kHistAlloc + kProbeBins,
    kCounterWords = kHistUpdate + kProbeBins,
};
constexpr int kReplicas = 64;

__device__ __forceinline__ unsigned long long* replica(unsigned long long* counters) {
    return counters + (size_t)(blockIdx.x % kReplicas) * kCounterWords;
}

// 16-byte table entry: packed key, pool index, 4 bytes of padding.
struct __align__(16) Entry {
    unsigned long long key;
    unsigned int idx;
    unsigned int pad;
};

constexpr unsigned int kNoSlot = 0xFFFFFFFFu;
constexpr unsigned int kSegOverflow = 0x80000000u;   // block's runs did not all fit: rescan it
constexpr float kNearPlane = 1e-4f;                 // block corners closer than this: whole image

// One run of a walk inside one block, as allocate records it for the
// update (12 bytes):
//   depth  the point's depth (f32 bits)
//   w1     colour R | G << 8 | B << 16, axis direction bits << 24 (bit set:
//          that axis steps by -1), cells - 1 << 27 (4 bits)
//   w2     first cell (voxel index in the block, 9 bits) | y-step plane << 9
//          (11 bits) | z-step plane << 20 (11 bits)
// The frame of the batch is the run's segment's (a filing holds one tile of
// one frame).  Bit q of the y-step (z-step) plane is set when the run's
// step q, the one from its cell q to cell q + 1, moves along y (z); a step
// with neither bit moves along x.  A run holds at most kMaxRunCells cells:
// the walk is monotonic on every axis and a block spans 8 cells per axis,
// so a walk's stretch through a block has at most 22 cells, and a stretch
// longer than kMaxRunCells is recorded as several runs of the same block.
// The update enumerates a run's cells from the record alone: it never
// repeats the walk's arithmetic.
struct RunRecord {
    unsigned int depth;
    unsigned int w1;
    unsigned int w2;
};
static_assert(sizeof(RunRecord) == 12, "12-byte run records");

constexpr int kMaxRunCells = 12;
constexpr int kPlaneBits = kMaxRunCells - 1;

__device__ __forceinline__ unsigned int run_w1(unsigned int colour_dirs, unsigned int cells) {
    return colour_dirs | ((cells - 1u) << 27);
}
__device__ __forceinline__ unsigned int run_w2(unsigned int entry, unsigned int ysteps, unsigned int zsteps) {
    return entry | (ysteps << 9) | (zsteps << (9 + kPlaneBits));
}
__device__ __forceinline__ int run_cells(unsigned int w1) { return (int)((w1 >> 27) & 15u) + 1; }
__device__ __forceinline__ int run_entry(unsigned int w2) { return (int)(w2 & 511u); }
__device__ __forceinline__ unsigned int run_ysteps(unsigned int w2) { return (w2 >> 9) & ((1u << kPlaneBits) - 1u); }
__device__ __forceinline__ unsigned int run_zsteps(unsigned int w2) {
    return (w2 >> (9 + kPlaneBits)) & ((1u << kPlaneBits) - 1u);
}

// A segment's position among its block's segments and the frame of its
// filing share a word (so do the runs before it and the frame in the
// block-ordered segment list): positions and run offsets below 2^25.
constexpr int kSegFrameShift = 25;
constexpr unsigned int kSegPosMask = (1u << kSegFrameShift) - 1u;

// One filing's runs through one block (an allocate workgroup's tile), as
// recorded by allocate.  One 64-bit atomic on the block's counter
// (segments << 32 | runs) gives both the segment's position among the
// block's segments and its first run's position among the block's runs, so
// in segment order block_off is the running total of the runs before it.
struct __align__(16) Segment {
    unsigned int slot;        // table slot of the block (kNoSlot: refused for lack of space)
    unsigned int rec_base;    // its first record in the record buffer
    unsigned int block_off;   // runs of the block's earlier segments
    unsigned int seg_pos;     // its position among the block's segments | frame << kSegFrameShift
};

// A block touched by the call, as the owner update reads it.
struct __align__(16) ItemDesc {
    unsigned long long key;
    unsigned int idx;         // pool index (>= capacity: none)
    unsigned int rec_count;   // runs | kSegOverflow: runs did not fit, rescan
    unsigned int seg_first;   // its first segment in the block-ordered segment list
    unsigned int seg_count;
    unsigned int slot;
    unsigned int units;       // work units the update splits the block's runs into (1: not split)
};

// Per-frame counters of the owner update, in the caller's scratch buffer,
// one set per frame parity.  Items and run records are reserved in
// kParts partitions (allocate workgroup w uses partition w mod kParts) so
// that no single counter takes every workgroup's atomic.  The update hands blocks
// out through one work counter per XCD, each in its own 128-byte line.
constexpr int kParts = 64;
constexpr int kXcds = 8;
constexpr int kFetchStride = 32;        // words between the XCDs' work counters
// One partition's counters, 128 bytes apart from the next partition's:
// atomics on one cache line are carried out one after another, so counters
// that many wavefronts add to must not share a line.
struct PartCounters {
    unsigned long long segrec;          // segments << 32 | records reserved
    unsigned int items;                 // blocks first touched
    unsigned int pad[29];
};
static_assert(sizeof(PartCounters) == 128, "one partition per 128 bytes");
struct FrameCounters {
    PartCounters part[kParts];
    unsigned int items_spill;           // blocks beyond their partition's share
    unsigned int items_total;           // all blocks (set when the blocks are placed)
    unsigned long long placed;          // segments given to blocks
    // Pool indices from here on were claimed after the last update placed
    // its blocks: no update has written those pool blocks since the pool was
    // cleared, so they still hold zeros (set by the previous call's placing
    // kernel; 0 after create and reset).
    unsigned long long pool_start;
    unsigned int n_rescan;              // blocks whose runs did not fit (rescanned)
    unsigned int front, back;           // items placed from the front (big blocks) and from the back
    unsigned int n_extra;               // work units beyond each split block's first
    unsigned int unit_runs;             // runs per work unit of a split block
    unsigned int pad[21];
    unsigned int fetch[kXcds * kFetchStride];   // next item of XCD x at fetch[x * kFetchStride]
};
static_assert(sizeof(FrameCounters) % 128 == 0, "FrameCounters keeps the work counters in their own lines");

// A block whose runs are many next to the call's total is split into work
// units of unit_runs runs (at least kMinUnitRuns), each taken by its own
// workgroup, which adds its sums into the pool with float atomics; the
// extra units are listed (at most kMaxUnits of them) and taken first.
constexpr unsigned int kMinUnitRuns = 256;
constexpr unsigned int kMaxUnits = 8192;

// Owner-update bookkeeping in the caller's scratch buffer.
struct OwnerArgs {
    FrameCounters* fc;         // [2] by frame parity
    unsigned int* items;       // [kParts * item_part_cap] first-touched slots, by partition
    unsigned int* items_spill; // [table entries] slots beyond a partition's share
    unsigned int* seg_first_of;  // [table entries] slot -> its first place in the segment list this call
                                 //   (kNoSlot: the block is rescanned)
    unsigned long long* blk_count;  // [table entries] segments << 32 | runs (| kSegOverflow) per slot
    unsigned int* rescan;      // [table entries] items whose runs did not fit
    ItemDesc* desc;            // [table entries] per item
    Segment* segs;             // [kParts * seg_part_cap] allocate order
    uint2* seg_list;           // [kParts * seg_part_cap] (rec_base, block_off | frame << kSegFrameShift),
                               //   grouped by block
    RunRecord* recs;           // [kParts * rec_part_cap] allocate order (read in place)
    uint2* units;              // [kMaxUnits] (item, chunk >= 1) of split blocks
    unsigned int unit_target;  // work units a call aims for (<= kMaxUnits): blocks with more
                               // runs than the call's runs / unit_target are split
    unsigned int item_part_cap, seg_part_cap, rec_part_cap;
    unsigned int parity;       // call serial & 1
    int build_items;           // 0: ray-parallel update, nothing recorded
};

// Per-launch frame arguments (passed by value; lands in SGPRs).
struct FrameArgs {
    const float* depth;
    const uint8_t* rgb;
    int width, height;
    float fx, fy, cx, cy;
    float R[9];
    float t[3];
    int max_visits;      // safety bound on one walk, >= any walk the frame can produce
    int tiles_x;         // 16 x 16 pixel tiles per row
    int n_tiles;
    int tiles_per_xcd;   // ceil(n_tiles / 8): workgroup -> tile remap
};

// The frames of one call (tsdf_integrate_batch, or one frame).  Frame i
// uses workgroups [i * tile_grid, (i + 1) * tile_grid) of the per-pixel
// kernels; tile_grid is a multiple of 8, so the workgroup -> XCD mapping is
// the same for every frame.  The first kArgFrames frames travel in the
// kernel arguments; the others (a call of more frames) in a device table
// the library fills before the call's kernels (`more`, frame kArgFrames
// first).
constexpr int kMaxBatch = 128;              // 7-bit frame index beside a segment's position
constexpr int kArgFrames = 32;
struct BatchArgs {
    FrameArgs f[kArgFrames];
    const FrameArgs* more;
    int n;
    int tile_grid;
};

// Where frame i of the batch is (kernel arguments or the device table).
__device__ __forceinline__ const FrameArgs* frame_ptr(const BatchArgs& b, int i) {
    return i < kArgFrames ? b.f + i : b.more + (i - kArgFrames);
}

// Frame i of the batch, i the same in every lane and every lane active: lane
// k loads the frame's word k and the wavefront reads each word into a
// scalar register (a plain load through frame_ptr would be one load per
// lane and field, the pointer being either of two memories).
__device__ __forceinline__ FrameArgs batch_frame(const BatchArgs& b, int i) {
    constexpr int kWords = (int)(sizeof(FrameArgs) / 4);
    static_assert(sizeof(FrameArgs) % 4 == 0 && kWords <= 64, "a frame's words fit a wavefront");
    const unsigned int* src = reinterpret_cast<const unsigned int*>(frame_ptr(b, i));
    const int lane = (int)(threadIdx.x & 63u);
    const unsigned int w = lane < kWords ? src[lane] : 0u;
    FrameArgs f;
    unsigned int* dst = reinterpret_cast<unsigned int*>(&f);
#pragma unroll
    for (int k = 0; k < kWords; ++k) dst[k] = (unsigned int)__builtin_amdgcn_readlane(w, k);
    return f;
}

// A pointer into memory that no kernel writes while it is read (the kernel
// arguments, the frame table), in the constant address space: a load through
// it at a wavefront-uniform address is a scalar load.
template <class T>
using ConstRef = const __attribute__((address_space(4))) T*;
template <class T>
__device__ __forceinline__ ConstRef<T> const_ref(const T* p) {
    return (ConstRef<T>)p;
}
// The same pointer, opaque to the optimiser: loads through the result happen
// where they are written, so a value needed at several places of a long
// kernel is loaded again (a few scalar loads) instead of being held in scalar
// registers in between (which, with the scalar register file full, spills it
// into lanes of a vector register: vector instructions for every use).
template <class T>
__device__ __forceinline__ ConstRef<T> reload(ConstRef<T> p) {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return p + __builtin_amdgcn_readfirstlane(z);
}

// The object a constant-address pointer points to (its fields are loaded
// where the copy's fields are used; unused fields are not loaded).
template <class T>
__device__ __forceinline__ T load_ref(ConstRef<T> p) {
    T v;
    __builtin_memcpy(&v, (const T*)p, sizeof(T));
    return v;
}

// Frame i of the batch as a constant-address pointer (i wavefront-uniform).
__device__ __forceinline__ ConstRef<FrameArgs> frame_ref(const BatchArgs& b, int i) {
    return i < kArgFrames ? const_ref(b.f + i) : const_ref(b.more + (i - kArgFrames));
}

struct VolumeArgs {
    Entry* table;
    unsigned int mask;               // table_entries - 1
    unsigned long long capacity;     // pool blocks
    float* tsdf;
    float* weight;
    float* r;
    float* g;
    float* b;
    unsigned long long* counters;
    float vs, inv_vs, trunc, inv_trunc;
    unsigned int probe_limit;        // slots a table operation may probe (0xFFFFFFFF: no limit)
    int reproject;                   // occlusion test: 0 the point's own depth, 1 also the depth image
};

enum PointClass { kInvalid = 0, kNear = 1, kOutside = 2, kValid = 3 };

// One point's walk through the unit voxel cells its band segment crosses.
struct BandWalk {
    float d;
    float gA0, gA1, gA2;
    float inv0, inv1, inv2;
    float tm0, tm1, tm2;
    int k0, k1, k2;
    int s0, s1, s2;
    // cells the walk can visit lie in [span_lo - 1, span_hi + 1] per axis
    // (the start and end cells, plus one for a final step that lands on a
    // boundary exactly)
    int span_lo0, span_lo1, span_lo2;
    int span_hi0, span_hi1, span_hi2;
};

__device__ __forceinline__ void setup_axis(float gA, float gB, int& k, int& s, float& inv, float& tm) {
    k = (int)floorf(gA);
    const float dir = gB - gA;
    // one division for both signs (a branch each would run both when the
    // lanes of a wavefront disagree)
    const float r = 1.0f / dir;
    s = dir > kStillAxis ? 1 : (dir < -kStillAxis ? -1 : 0);
    inv = s != 0 ? r : 0.0f;
    tm = s > 0 ? ((float)(k + 1) - gA) * r : (s < 0 ? ((float)k - gA) * r : __builtin_inff());
}

// Classify pixel (u, v) with depth d and, for a valid point, set up its walk.
// The band is the camera-z interval [d - trunc, d + trunc] along the pixel
// ray, mapped to the world by the pose and to voxel units by 1/vs.
// Every field is computed for every pixel, whatever its class (no branches:
// the lanes of a wavefront need no masking); a pixel whose class is not
// kValid gets values that must not be used.
// xn = (u - cx) / fx and yn = (v - cy) / fy are the pixel ray's slopes
// (callers that share them between pixels compute them once).
__device__ __forceinline__ int setup_walk(BandWalk& w, float d, float xn, float yn, const FrameArgs& f,
                                          float trunc, float inv_vs) {
    const float z0 = d - trunc;
    const float z1 = d + trunc;
    const float a0 = xn * z0, a1 = yn * z0, a2 = z0;
    const float b0 = xn * z1, b1 = yn * z1, b2 = z1;
    const float gA0 = (((f.R[0] * a0 + f.R[1] * a1) + f.R[2] * a2) + f.t[0]) * inv_vs;
    const float gA1 = (((f.R[3] * a0 + f.R[4] * a1) + f.R[5] * a2) + f.t[1]) * inv_vs;
    const float gA2 = (((f.R[6] * a0 + f.R[7] * a1) + f.R[8] * a2) + f.t[2]) * inv_vs;
    const float gB0 = (((f.R[0] * b0 + f.R[1] * b1) + f.R[2] * b2) + f.t[0]) * inv_vs;
    const float gB1 = (((f.R[3] * b0 + f.R[4] * b1) + f.R[5] * b2) + f.t[1]) * inv_vs;
    const float gB2 = (((f.R[6] * b0 + f.R[7] * b1) + f.R[8] * b2) + f.t[2]) * inv_vs;
    // keys hold +-2^20 blocks per axis; keep every visited cell inside that
    const bool in_range = fabsf(gA0) <= kRangeLimit && fabsf(gA1) <= kRangeLimit &&
                          fabsf(gA2) <= kRangeLimit && fabsf(gB0) <= kRangeLimit &&
                          fabsf(gB1) <= kRangeLimit && fabsf(gB2) <= kRangeLimit;
    w.d = d;
    w.gA0 = gA0;
    w.gA1 = gA1;
    w.gA2 = gA2;
    setup_axis(gA0, gB0, w.k0, w.s0, w.inv0, w.tm0);
    setup_axis(gA1, gB1, w.k1, w.s1, w.inv1, w.tm1);
    setup_axis(gA2, gB2, w.k2, w.s2, w.inv2, w.tm2);
    const int e0 = (int)floorf(gB0), e1 = (int)floorf(gB1), e2 = (int)floorf(gB2);
    w.span_lo0 = min(w.k0, e0);
    w.span_lo1 = min(w.k1, e1);
    w.span_lo2 = min(w.k2, e2);
    w.span_hi0 = max(w.k0, e0);
    w.span_hi1 = max(w.k1, e1);
    w.span_hi2 = max(w.k2, e2);
    if (!__builtin_isfinite(d) || !(d > 0.0f)) return kInvalid;
    if (d <= trunc) return kNear;
    return in_range ? kValid : kOutside;
}
__device__ __forceinline__ int setup_walk(BandWalk& w, float d, int u, int v, const FrameArgs& f,
                                          float trunc, float inv_vs) {
    return setup_walk(w, d, ((float)u - f.cx) / f.fx, ((float)v - f.cy) / f.fy, f, trunc, inv_vs);
}

// The lane's own bit of a wavefront lane mask, as its condition.
__device__ __forceinline__ bool lane_on(unsigned long long mask) { return __builtin_amdgcn_inverse_ballot_w64(mask); }

// x + x + (this lane's bit of mask): one add with the mask as carry-in.
__device__ __forceinline__ unsigned int shift_in(unsigned int x, unsigned long long mask) {
    unsigned int r;
    unsigned long long carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(x), "s"(mask));
    return r;
}
// x + (this lane's bit of mask), the same way
__device__ __forceinline__ unsigned int count_in(unsigned int x, unsigned long long mask) {
    unsigned int r;
    unsigned long long carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, 0, %3" : "=v"(r), "=s"(carry_out) : "v"(x), "s"(mask));
    return r;
}

// Occlusion and band test at the centre of the current cell.  sdf is the
// observed depth minus the camera depth of the centre; keep iff
// -trunc <= sdf <= trunc (a centre further behind the surface is hidden).
__device__ __forceinline__ bool centre_test(const BandWalk& w, const FrameArgs& f, float vs, float trunc,
                                            float& sdf) {
    const float c0 = ((float)w.k0 + 0.5f) * vs;
    const float c1 = ((float)w.k1 + 0.5f) * vs;
    const float c2 = ((float)w.k2 + 0.5f) * vs;
    const float zc = (f.R[2] * (c0 - f.t[0]) + f.R[5] * (c1 - f.t[1])) + f.R[8] * (c2 - f.t[2]);
    sdf = w.d - zc;
    return sdf >= -trunc && sdf <= trunc;
}

// The same test with the pose's third column and the translation held in
// registers (callers whose frame lives in LDS load them once per walk).
struct DepthAxis {
    float r2, r5, r8, t0, t1, t2;
};

__device__ __forceinline__ DepthAxis depth_axis(const FrameArgs& f) {
    DepthAxis a;
    a.r2 = f.R[2];
    a.r5 = f.R[5];
    a.r8 = f.R[8];
    a.t0 = f.t[0];
    a.t1 = f.t[1];
    a.t2 = f.t[2];
    return a;
}


// The same test for cell (k0, k1, k2) of a point with depth d.
// The centre test from the centre's coordinates in voxels, (float)k + 0.5f
// per axis (the walk keeps them exactly, see k_allocate).
__device__ __forceinline__ bool centre_test_at(float x, float y, float z, float d, const DepthAxis& a, float vs,
                                               float trunc, float& sdf) {
    const float c0 = x * vs;
    const float c1 = y * vs;
    const float c2 = z * vs;
    const float zc = (a.r2 * (c0 - a.t0) + a.r5 * (c1 - a.t1)) + a.r8 * (c2 - a.t2);
    sdf = d - zc;
    return sdf >= -trunc && sdf <= trunc;
}
__device__ __forceinline__ bool centre_test(int k0, int k1, int k2, float d, const DepthAxis& a, float vs,
                                            float trunc, float& sdf) {
    return centre_test_at((float)k0 + 0.5f, (float)k1 + 0.5f, (float)k2 + 0.5f, d, a, vs, trunc, sdf);
}

// The reprojection reading of the occlusion test: what a frame contributes
// to it (the camera's x and y axes in world coordinates, i.e. columns 0 and 1
// of the rotation, the intrinsics and the depth image).
struct Projection {
    float rx0, rx1, rx2;      // R[0][0], R[1][0], R[2][0]
    float ry0, ry1, ry2;      // R[0][1], R[1][1], R[2][1]
    float fx, fy, cx, cy;
    float fw, fh;             // image width and height
    const float* depth;
    int width;
};

__device__ __forceinline__ Projection projection(const FrameArgs& f) {
    Projection p;
    p.rx0 = f.R[0];
    p.rx1 = f.R[3];
    p.rx2 = f.R[6];
    p.ry0 = f.R[1];
    p.ry1 = f.R[4];
    p.ry2 = f.R[7];
    p.fx = f.fx;
    p.fy = f.fy;
    p.cx = f.cx;
    p.cy = f.cy;
    p.fw = (float)f.width;
    p.fh = (float)f.height;
    p.depth = f.depth;
    p.width = f.width;
    return p;
}

// Is a voxel centre (q = centre - camera position, camera depth zc) hidden
// behind the surface the depth image shows along its own line of sight?
// It projects to ((x / zc) fx + cx, (y / zc) fy + cy) in pixel units; the
// pixel whose centre is nearest (floor of coordinate + 0.5) holds depth D.
// Hidden iff that pixel is inside the image, D is finite and > 0, and the
// centre lies more than trunc behind it; a centre at or behind the camera
// plane, or with no valid depth at its pixel, is not hidden.
__device__ __forceinline__ bool hidden_in_image(float q0, float q1, float q2, float zc, const Projection& p,
                                                float trunc) {
    if (!(zc > 0.0f)) return false;
    const float x = (p.rx0 * q0 + p.rx1 * q1) + p.rx2 * q2;
    const float y = (p.ry0 * q0 + p.ry1 * q1) + p.ry2 * q2;
    const float uf = ((x / zc) * p.fx + p.cx) + 0.5f;
    const float vf = ((y / zc) * p.fy + p.cy) + 0.5f;
    if (!(uf >= 0.0f && uf < p.fw && vf >= 0.0f && vf < p.fh)) return false;
    const float D = p.depth[(size_t)(unsigned int)floorf(vf) * (unsigned int)p.width + (unsigned int)floorf(uf)];
    if (!__builtin_isfinite(D) || !(D > 0.0f)) return false;
    return zc - D > trunc;
}

// centre_test with the reprojection reading added (same centre arithmetic).
__device__ __forceinline__ bool centre_test_reproject_at(float x, float y, float z, float d, const DepthAxis& a,
                                                         const Projection& p, float vs, float trunc, float& sdf) {
    const float q0 = (x * vs) - a.t0;
    const float q1 = (y * vs) - a.t1;
    const float q2 = (z * vs) - a.t2;
    const float zc = (a.r2 * q0 + a.r5 * q1) + a.r8 * q2;
    sdf = d - zc;
    return sdf >= -trunc && sdf <= trunc && !hidden_in_image(q0, q1, q2, zc, p, trunc);
}
__device__ __forceinline__ bool centre_test_reproject(int k0, int k1, int k2, float d, const DepthAxis& a,
                                                      const Projection& p, float vs, float trunc, float& sdf) {
    return centre_test_reproject_at((float)k0 + 0.5f, (float)k1 + 0.5f, (float)k2 + 0.5f, d, a, p, vs, trunc,
                                    sdf);
}

// Step to the next cell: the axis with the smallest boundary parameter (ties
// to x, then y), until that parameter passes the segment end (1).
__device__ __forceinline__ bool advance(BandWalk& w) {
    float tmin = w.tm0;
    int m = 0;
    if (w.tm1 < tmin) {
        tmin = w.tm1;
        m = 1;
    }
    if (w.tm2 < tmin) {
        tmin = w.tm2;
        m = 2;
    }
    if (!(tmin <= 1.0f)) return false;
    if (m == 0) {
        w.k0 += w.s0;
        w.tm0 = ((float)(w.s0 > 0 ? w.k0 + 1 : w.k0) - w.gA0) * w.inv0;
    } else if (m == 1) {
        w.k1 += w.s1;
        w.tm1 = ((float)(w.s1 > 0 ? w.k1 + 1 : w.k1) - w.gA1) * w.inv1;
    } else {
        w.k2 += w.s2;
        w.tm2 = ((float)(w.s2 > 0 ? w.k2 + 1 : w.k2) - w.gA2) * w.inv2;
    }
    return true;
}

// advance() without branches: the same choice of axis (smallest boundary
// parameter, ties to x, then y) and the same recomputation, done with
// selects so the lanes of a wavefront never split on the axis.  Returns
// false, leaving the walk unchanged, when the walk ends; otherwise sets
// `crossed` if the step left the 8^3 block of the previous cell, and `axis`
// to the axis stepped.
// (Every operand of the selects below is a prvalue: a conditional between
// two lvalue fields of the walk would select between their addresses and
// keep the whole walk in scratch memory.)
template <typename T>
__device__ __forceinline__ T value_of(const T& x) {
    return x;
}

__device__ __forceinline__ bool advance_select(BandWalk& w, bool& crossed, int& axis) {
    const float tm0 = value_of(w.tm0), tm1 = value_of(w.tm1), tm2 = value_of(w.tm2);
    const int k0 = value_of(w.k0), k1 = value_of(w.k1), k2 = value_of(w.k2);
    const bool c1 = tm1 < tm0;
    const float t01 = c1 ? (float)tm1 : (float)tm0;
    const bool c2 = tm2 < t01;
    const float tmin = c2 ? (float)tm2 : (float)t01;
    const bool more = tmin <= 1.0f;
    const bool a2 = more && c2;
    const bool a1 = more && !c2 && c1;
    const bool a0 = more && !c2 && !c1;
    const int s0 = value_of(w.s0), s1 = value_of(w.s1), s2 = value_of(w.s2);
    const float g0 = value_of(w.gA0), g1 = value_of(w.gA1), g2 = value_of(w.gA2);
    const float i0 = value_of(w.inv0), i1 = value_of(w.inv1), i2 = value_of(w.inv2);
    const int k_old = c2 ? (int)k2 : (c1 ? (int)k1 : (int)k0);
    const int s = c2 ? (int)s2 : (c1 ? (int)s1 : (int)s0);
    const float gA = c2 ? (float)g2 : (c1 ? (float)g1 : (float)g0);
    const float inv = c2 ? (float)i2 : (c1 ? (float)i1 : (float)i0);
    const int k = k_old + s;
    const float t = ((float)(s > 0 ? k + 1 : k) - gA) * inv;
    w.k0 = a0 ? k : k0;
    w.k1 = a1 ? k : k1;
    w.k2 = a2 ? k : k2;
    w.tm0 = a0 ? t : tm0;
    w.tm1 = a1 ? t : tm1;
    w.tm2 = a2 ? t : tm2;
    crossed = more && (k >> 3) != (k_old >> 3);
    axis = c2 ? 2 : (c1 ? 1 : 0);
    return more;
}

// 64-bit key: block coordinate (cell >> 3, i.e. floor(cell / 8)) + 2^20 per
// axis, x in bits 0-20, y in 21-41, z in 42-62; bit 63 stays clear, so no
// key equals the empty marker.
__device__ __forceinline__ unsigned long long block_key(int k0, int k1, int k2) {
    return (unsigned long long)(unsigned int)((k0 >> 3) + kKeyBias) |
           ((unsigned long long)(unsigned int)((k1 >> 3) + kKeyBias) << 21) |
           ((unsigned long long)(unsigned int)((k2 >> 3) + kKeyBias) << 42);
}

__device__ __forceinline__ int voxel_in_block(int k0, int k1, int k2) {
    return (k0 & 7) | ((k1 & 7) << 3) | ((k2 & 7) << 6);
}

// Multiply-xor hash of the key (the 64-bit finaliser of MurmurHash3),
// reduced to a home slot.
__device__ __forceinline__ unsigned int home_slot(unsigned long long key, unsigned int mask) {
    key ^= key >> 33;
    key *= 0xff51afd7ed558ccdull;
    key ^= key >> 33;
    key *= 0xc4ceb9fe1a85ec53ull;
    key ^= key >> 33;
    return (unsigned int)key & mask;
}

// Make sure `key` is in the table.  Linear probing from its home slot with
// no fixed bound: it ends at the key, at an empty slot won by the one 64-bit
// compare-exchange, or after every slot was tried (counted as table_full).
// Keys are read with plain loads: a slot only ever goes from empty to a
// key, so a stale empty read just leads to a compare-exchange whose returned
// value is authoritative.  Returns the slot (kNoSlot if the table is full);
// `won` tells whether this call inserted the key (the caller then takes a
// pool index for it and publishes it), `probes` the slots probed.
__device__ __forceinline__ unsigned int insert_key(const VolumeArgs& vol, unsigned long long key, bool& won,
                                                   unsigned int& probes) {
    unsigned int slot = home_slot(key, vol.mask);
    probes = 1;
    won = false;
    for (;;) {
        const unsigned long long cur = vol.table[slot].key;
        if (cur == key) return slot;
        if (cur == kEmptyKey) {
            const unsigned long long prev = atomicCAS(&vol.table[slot].key, kEmptyKey, key);
            if (prev == kEmptyKey) {
                won = true;
                return slot;
            }
            if (prev == key) return slot;
        }
        if (probes > vol.mask) {       // every slot tried
            atomicAdd(replica(vol.counters) + kTableFull, 1ull);
            return kNoSlot;
        }
        if (probes >= vol.probe_limit) {   // the bounded-probe control gives up here
            atomicAdd(replica(vol.counters) + kProbeExhausted, 1ull);
            return kNoSlot;
        }
        slot = (slot + 1) & vol.mask;
        ++probes;
    }
}

// Lane 0's value, as a wavefront-uniform scalar (lane 0 must be active).
__device__ __forceinline__ unsigned int read_lane0(unsigned int x) { return __builtin_amdgcn_readlane(x, 0); }
__device__ __forceinline__ unsigned long long read_lane0(unsigned long long x) {
    return ((unsigned long long)__builtin_amdgcn_readlane((unsigned int)(x >> 32), 0) << 32) |
           (unsigned int)__builtin_amdgcn_readlane((unsigned int)x, 0);
}

// The lanes of a wavefront that inserted keys take consecutive pool indices
// with one atomic, and publish them (kNoIndex once the pool is full).  Must
// be called by the whole wavefront.
__device__ __forceinline__ void claim_pool_indices(const VolumeArgs& vol, bool won, unsigned int slot) {
    const unsigned long long m = __ballot(won);
    if (!m) return;
    const int lane = threadIdx.x & 63;
    unsigned long long base = 0;
    if (lane == 0) base = atomicAdd(vol.counters + kBlockCounter, (unsigned long long)__popcll(m));
    base = read_lane0(base);
    if (won) {
        const unsigned long long idx = base + (unsigned long long)__popcll(m & ((1ull << lane) - 1ull));
        const unsigned int pub = idx < vol.capacity ? (unsigned int)idx : kNoIndex;
        __hip_atomic_store(&vol.table[slot].idx, pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Look `key` up after allocation has completed (a kernel boundary earlier on
// the stream): returns its pool index, or kNoIndex if the key is absent or
// was refused a pool index.
__device__ __forceinline__ unsigned int lookup_key(const VolumeArgs& vol, unsigned long long key,
                                                   unsigned int& probes) {
    unsigned int slot = home_slot(key, vol.mask);
    probes = 1;
    for (;;) {
        const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(vol.table + slot);
        if (e.x == key) {
            const unsigned int idx = (unsigned int)e.y;
            return idx < vol.capacity ? idx : kNoIndex;
        }
        if (e.x == kEmptyKey || probes > vol.mask) return kNoIndex;
        if (probes >= vol.probe_limit) {
            atomicAdd(replica(vol.counters) + kProbeExhausted, 1ull);
            return kNoIndex;
        }
        slot = (slot + 1) & vol.mask;
        ++probes;
    }
}

// Sum over the wavefront (every lane active): DPP row operations, no LDS.
__device__ __forceinline__ unsigned int wave_sum(unsigned int x) { return __reduce_add_sync(~0ull, x); }

// Inclusive prefix sum over the wavefront's lanes (every lane active).
// Does any active lane hold b?  (The ballot of the lane mask itself: no
// detour through a 0/1 value in a vector register.)
__device__ __forceinline__ bool wave_any(bool b) { return __builtin_amdgcn_ballot_w64(b) != 0; }

__device__ __forceinline__ unsigned int wave_inclusive_sum(unsigned int x) {
    const int lane = (int)(threadIdx.x & 63u);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned int y = __shfl_up(x, (unsigned int)d);
        x += lane >= d ? y : 0u;
    }
    return x;
}

__device__ __forceinline__ void unpack_key(unsigned long long key, int& bx, int& by, int& bz) {
    bx = (int)(key & 0x1FFFFFull) - kKeyBias;
    by = (int)((key >> 21) & 0x1FFFFFull) - kKeyBias;
    bz = (int)((key >> 42) & 0x1FFFFFull) - kKeyBias;
}

// Pixels (inclusive rectangle) whose band can reach block (bx, by, bz), and
// the camera-depth range of that reach.  The block's cells grown by one cell
// on every side (covering rounding of the walk at cell boundaries) are
// projected corner by corner; every point of a pixel's band segment projects
// to that pixel, so a pixel whose walk enters the block lies in the bounding
// box of the corner projections, widened by one pixel for rounding.  A box
// reaching the camera plane covers the whole image.
struct PixelRect {
    int u0, v0, u1, v1;
    float zmin, zmax;
};

__device__ __forceinline__ PixelRect block_rect(int bx, int by, int bz, const FrameArgs& f, float vs) {
    const float lo[3] = {(float)(8 * bx - 1) * vs, (float)(8 * by - 1) * vs, (float)(8 * bz - 1) * vs};
    const float hi[3] = {(float)(8 * bx + 9) * vs, (float)(8 * by + 9) * vs, (float)(8 * bz + 9) * vs};
    float umin = __builtin_inff(), umax = -__builtin_inff();
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    float zmin = __builtin_inff(), zmax = -__builtin_inff();
    bool behind = false;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float d0 = ((c & 1) ? hi[0] : lo[0]) - f.t[0];
        const float d1 = ((c & 2) ? hi[1] : lo[1]) - f.t[1];
        const float d2 = ((c & 4) ? hi[2] : lo[2]) - f.t[2];
        const float xc = f.R[0] * d0 + f.R[3] * d1 + f.R[6] * d2;
        const float yc = f.R[1] * d0 + f.R[4] * d1 + f.R[7] * d2;
        const float zc = f.R[2] * d0 + f.R[5] * d1 + f.R[8] * d2;
        zmin = fminf(zmin, zc);
        zmax = fmaxf(zmax, zc);
        if (!(zc > kNearPlane)) {
            behind = true;
        } else {
            const float u = f.fx * (xc / zc) + f.cx;
            const float v = f.fy * (yc / zc) + f.cy;
            umin = fminf(umin, u);
            umax = fmaxf(umax, u);
            vmin = fminf(vmin, v);
            vmax = fmaxf(vmax, v);
        }
    }
    PixelRect r;
    r.zmin = zmin;
    r.zmax = zmax;
    if (behind) {
        r.u0 = 0;
        r.v0 = 0;
        r.u1 = f.width - 1;
        r.v1 = f.height - 1;
        return r;
    }
    const float W = (float)f.width, H = (float)f.height;
    r.u0 = (int)floorf(fminf(fmaxf(umin, -2.0f), W + 2.0f)) - 1;
    r.u1 = (int)ceilf(fminf(fmaxf(umax, -2.0f), W + 2.0f)) + 1;
    r.v0 = (int)floorf(fminf(fmaxf(vmin, -2.0f), H + 2.0f)) - 1;
    r.v1 = (int)ceilf(fminf(fmaxf(vmax, -2.0f), H + 2.0f)) + 1;
    r.u0 = max(r.u0, 0);
    r.v0 = max(r.v0, 0);
    r.u1 = min(r.u1, f.width - 1);
    r.v1 = min(r.v1, f.height - 1);
    return r;
}


}  // namespace tsdf
