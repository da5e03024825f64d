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

// Counter words (uint64) at the start of the caller's counters buffer.
enum CounterWord {
    kBlockCounter = 0,   // next pool index; may run past the capacity
    kTableFull,
    kUpdateMisses,
    kOutOfRange,
    kNearSkipped,
    kPointsValid,
    kVoxelUpdates,
    kWalkGuard,
    kProbeMax,
    kHistAlloc = 16,
    kHistUpdate = kHistAlloc + kProbeBins,
    kCounterWords = kHistUpdate + kProbeBins,
};

struct __align__(16) Entry {
    unsigned long long key;
    unsigned int idx;
    unsigned int pad;
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
};

__device__ __forceinline__ void setup_axis(float gA, float gB, int& k, int& s, float& inv, float& tm) {
    k = (int)floorf(gA);
    const float dir = gB - gA;
    if (dir > kStillAxis) {
        s = 1;
        inv = 1.0f / dir;
        tm = ((float)(k + 1) - gA) * inv;
    } else if (dir < -kStillAxis) {
        s = -1;
        inv = 1.0f / dir;
        tm = ((float)k - gA) * inv;
    } else {
        s = 0;
        inv = 0.0f;
        tm = __builtin_inff();
    }
}

// Classify pixel (u, v) with depth d and, for a valid point, set up its walk.
// The band is the camera-z interval [d - trunc, d + trunc] along the pixel
// ray, mapped to the world by the pose and to voxel units by 1/vs.
__device__ __forceinline__ int setup_walk(BandWalk& w, float d, int u, int v, const FrameArgs& f,
                                          float trunc, float inv_vs) {
    if (!__builtin_isfinite(d) || !(d > 0.0f)) return kInvalid;
    if (d <= trunc) return kNear;
    const float xn = ((float)u - f.cx) / f.fx;
    const float yn = ((float)v - f.cy) / f.fy;
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
    if (!in_range) return kOutside;
    w.d = d;
    w.gA0 = gA0;
    w.gA1 = gA1;
    w.gA2 = gA2;
    setup_axis(gA0, gB0, w.k0, w.s0, w.inv0, w.tm0);
    setup_axis(gA1, gB1, w.k1, w.s1, w.inv1, w.tm1);
    setup_axis(gA2, gB2, w.k2, w.s2, w.inv2, w.tm2);
    return kValid;
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
// The winner takes the next pool index and publishes it (or kNoIndex once
// the pool is full).  Keys are read with plain loads: a slot only ever goes
// from empty to a key, so a stale empty read just leads to a compare-exchange
// whose returned value is authoritative.  Returns the slots probed.
__device__ __forceinline__ unsigned int insert_key(const VolumeArgs& vol, unsigned long long key) {
    unsigned int slot = home_slot(key, vol.mask);
    unsigned int probes = 1;
    for (;;) {
        const unsigned long long cur = vol.table[slot].key;
        if (cur == key) break;
        if (cur == kEmptyKey) {
            const unsigned long long prev = atomicCAS(&vol.table[slot].key, kEmptyKey, key);
            if (prev == kEmptyKey) {
                const unsigned long long idx = atomicAdd(vol.counters + kBlockCounter, 1ull);
                const unsigned int pub = idx < vol.capacity ? (unsigned int)idx : kNoIndex;
                __hip_atomic_store(&vol.table[slot].idx, pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            if (prev == key) break;
        }
        if (probes > vol.mask) {       // every slot tried
            atomicAdd(vol.counters + kTableFull, 1ull);
            break;
        }
        slot = (slot + 1) & vol.mask;
        ++probes;
    }
    return probes;
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
        slot = (slot + 1) & vol.mask;
        ++probes;
    }
}

__device__ __forceinline__ unsigned int wave_sum(unsigned int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace tsdf
