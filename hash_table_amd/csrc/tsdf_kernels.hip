// tsdf_kernels.hip -- gfx950 kernels of the integrate path and their host
// launch wrappers (declared in tsdf_kernels.hpp).
//
// The integrate path of hash-blocked TSDF fusion as "What Irregularity
// Costs: CUDA C++, Rust, and Triton on a Hash-Blocked GPU Workload"
// describes it in section 3: two kernels over the same points, `allocate`
// (the irregular stage: probe, compare-exchange, insert) and `update` (the
// regular stage: accumulate sums into the blocks).  Both apply the same
// occlusion test and produce the same per-voxel sums; how the update is
// organised is this library's choice for the MI355X memory system:
//
//   * owner update (default): allocate cuts every walk into runs, one per
//     block it crosses, and records each run with a kept voxel (depth,
//     colour, first cell and the axis of each step: 12 bytes; the frame goes
//     with the run's segment); the records are grouped by block, and one
//     workgroup per block enumerates the cells of each of its runs (no walk
//     arithmetic repeated), sums the block's contributions in LDS and then
//     read-modify-writes the five pool arrays with plain coalesced loads and
//     stores: a block has one writer per call, so no device-scope float
//     atomics are needed.  A block
//     whose runs did not fit the record buffers is rescanned from the pixel
//     rectangle its band can be seen through.
//   * ray-parallel update: the shape the paper describes (one thread per
//     point, a lookup per block run, five no-return f32 atomic additions per
//     voxel), kept as a variant.
//
// Launch geometry of the per-point kernels: one thread per pixel; a
// 256-thread workgroup (four wave64 wavefronts) covers a 16 x 16 tile, each
// wavefront an 8 x 8 sub-tile, so a wave's rays mostly touch the same blocks.
// Workgroups go to the eight XCDs round-robin; the workgroup -> tile remap
// gives each XCD a contiguous run of tiles so neighbouring tiles share an L2.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tsdf_kernels.hpp"

namespace tsdf {
namespace {

constexpr int kTile = 16;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kInv255 = 1.0f / 255.0f;
constexpr int kChunkCells = 31;   // cells of a walk per pass of the allocate loop (plus a sentinel bit)

__device__ __forceinline__ bool workgroup_tile(const FrameArgs& f, int wg, int& tile_u0, int& tile_v0) {
    const int rank = wg / kXcds;                   // position within the XCD's run of tiles
    if (rank >= f.tiles_per_xcd) return false;     // a smaller frame of the batch
    const int tile = (wg % kXcds) * f.tiles_per_xcd + rank;
    if (tile >= f.n_tiles) return false;
    tile_u0 = (tile % f.tiles_x) * kTile;
    tile_v0 = (tile / f.tiles_x) * kTile;
    return true;
}

// One of three values by two conditions.  (Taking the values, not
// references: a conditional over references to a lambda's captures would
// select between their addresses and keep the variables in memory.)
__device__ __forceinline__ float pick3(bool first, bool second, float a, float b, float c) {
    return first ? a : (second ? b : c);
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
    unsigned long long* c = replica(counters);
    if (t < kProbeBins && s_hist[t]) atomicAdd(c + base + t, (unsigned long long)s_hist[t]);
    if (t == kProbeBins && *s_pmax) atomicMax(c + kProbeMax, (unsigned long long)*s_pmax);
}

// ---------------------------------------------------------------------------
// allocate.  Each lane walks its ray in chunks of up to kChunkCells cells and
// cuts each chunk into runs, one per block the walk crosses; a lane holds
// its runs with a kept voxel in kSlots register slots.  Full slots (or the
// end of the chunk) are filed for the whole workgroup (the 16 x 16 tile) at
// once: the run keys go into an LDS hash set, whose per-key run counter
// hands each run its rank among the key's runs; one thread per distinct key
// probes the global table and adds the key's runs to its block counter, one
// reservation takes the filing's segments (one per distinct key) and
// records, and every lane then writes the records of its own runs at the
// key's base + rank.  Neighbouring rays cross the same few blocks, so a
// workgroup's filing has few distinct keys and each segment holds many runs.
// Also counts the point classes and the kept (point, voxel) pairs.
// ---------------------------------------------------------------------------
constexpr int kSlots = 4;                         // runs a lane holds between filings
constexpr int kSetCap = kSlots * kThreads;        // LDS set: room for every run of a filing
constexpr int kSetBits = 10;
static_assert(kSetCap == 1 << kSetBits, "set_slot yields kSetBits bits");
constexpr unsigned int kNoBase = 0xFFFFFFFFu;     // runs not recorded (block rescanned)
constexpr unsigned int kNoKeyBase = 0xFFFFFFFEu;  // runs of a key the full table refused

struct AllocLds {
    unsigned long long skey[kSetCap];             // set: key (empty: all ones),
    unsigned int scnt[kSetCap];                   //   its runs; after the reservation, its first record
    unsigned short sslot[kSetCap];                // set slots of the distinct keys, in insertion order
    unsigned long long scode[kSlots][kThreads];   // the lanes' RunSlots codes, held here while the keys are filed
    unsigned long long r0;                        // the filing's reservation: first segment << 32 | first record
    unsigned int nuniq;                           // distinct keys of the filing
    unsigned int nrun;                            // its runs
    unsigned int nrec;                            // records handed to its keys so far
    unsigned int votes[3];                        // workgroup_any, in rotation
    unsigned int hist[kProbeBins];
    unsigned int pmax;
    unsigned int cnt[6];
    float xn[kTile], yn[kTile];                   // the tile's pixel-ray slopes per column and row
};

// A lane's runs since the last filing: slot q holds its q-th run (pend: a
// run with a kept voxel waiting to be filed): its block key, and its
// record's w2 with the cell count and the kept cells above it
// (w2 | (cells | kept << 8) << 32).
struct RunSlots {
    unsigned long long key[kSlots];
    unsigned long long code[kSlots];
    bool pend[kSlots];
};

// Home slot of a block key in the LDS set (multiply-xor of the key's halves).
__device__ __forceinline__ unsigned int set_slot(unsigned long long key) {
    const unsigned int lo = (unsigned int)key, hi = (unsigned int)(key >> 32);
    return ((lo * 0x9E3779B1u) ^ (hi * 0x85EBCA77u)) >> (32 - kSetBits);
}

// Whether p holds in any thread of the workgroup (one barrier).  Every
// thread calls it with the same rnd, which it advances: call k votes in word
// k mod 3 and clears the word of call k - 1 (read by every thread before
// this call's barrier; written again only after the next call's).
__device__ __forceinline__ bool workgroup_any(bool p, AllocLds& L, unsigned int& rnd) {
    const unsigned int r = rnd % 3u;
    if (__ballot(p) && (threadIdx.x & 63) == 0) L.votes[r] = 1u;
    __syncthreads();
    const bool any = L.votes[r] != 0u;
    if (threadIdx.x == 0) L.votes[(r + 2u) % 3u] = 0u;
    ++rnd;
    return any;
}

// File the workgroup's pending runs (see above).  depth and colour_dirs:
// this thread's point, for the records of its runs; frame: the workgroup's
// frame of the batch, for its segments.  Must be called by the whole
// workgroup after a barrier; the LDS set is empty on entry and again once the
// next barrier has passed.
__device__ __forceinline__ void file_runs(RunSlots& S, AllocLds& L, unsigned int part, ConstRef<VolumeArgs> vref,
                                          ConstRef<OwnerArgs> oref, unsigned int depth, unsigned int colour_dirs,
                                          unsigned int frame) {
    const VolumeArgs vol = load_ref(reload(vref));         // (loaded per filing, not held through the walk)
    const OwnerArgs own = load_ref(reload(oref));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // de-duplicate: each pending run finds (or enters) its key in the set
    // and takes a rank among the key's runs
    unsigned int hr[kSlots];                      // per run: set slot | rank << kSetBits
    unsigned int wave_runs = 0;
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
        hr[q] = 0;
        const unsigned long long pm = __ballot(S.pend[q]);
        if (!pm) continue;
        wave_runs += (unsigned int)__popcll(pm);
        if (S.pend[q]) {
            const unsigned long long key = S.key[q];
            unsigned int h = set_slot(key);
            for (;;) {     // at most kSetCap distinct keys: the probe always finds room
                const unsigned long long prev = atomicCAS(&L.skey[h], kEmptyKey, key);
                if (prev == kEmptyKey) {
                    L.sslot[atomicAdd(&L.nuniq, 1u)] = (unsigned short)h;
                    break;
                }
                if (prev == key) break;
                h = (h + 1) & (kSetCap - 1);
            }
            hr[q] = h | (atomicAdd(&L.scnt[h], 1u) << kSetBits);
            L.scode[q][tid] = S.code[q];
        }
    }
    if (wave_runs && lane == 0) atomicAdd(&L.nrun, wave_runs);
    __syncthreads();
    const unsigned int nu = L.nuniq;
    const unsigned long long below = (1ull << lane) - 1ull;
    FrameCounters* fc = own.fc + own.parity;      // owner mode only
    // one reservation for the filing: a segment per distinct key (key d
    // takes the d-th) and a record per run (its return is awaited only
    // where the segments are written)
    unsigned long long r0 = 0;
    if (own.build_items && tid == 0 && nu)
        r0 = atomicAdd(&fc->part[part].segrec, ((unsigned long long)nu << 32) | L.nrun);
    for (unsigned int d0 = 0; d0 < nu; d0 += kThreads) {   // workgroup-uniform: kThreads keys at a time
        const unsigned int d = d0 + (unsigned int)tid;
        const bool has = d < nu;
        unsigned int h = 0, slot = kNoSlot, runs = 0, roff = 0;
        unsigned long long bc = 0;
        if (d0 + (unsigned int)wave * 64u < nu) {           // (wavefront-uniform) this wavefront holds keys
            bool won = false;
            if (has) {
                h = L.sslot[d];
                unsigned int probes;
                slot = insert_key(vol, L.skey[h], won, probes);
                hist_add(L.hist, &L.pmax, probes);
            }
            claim_pool_indices(vol, won, slot);
            if (own.build_items) {
                // Each block's counter (segments << 32 | runs) takes one add
                // per filing.  The workgroup that finds it at zero is the
                // first to touch the block in this call and lists it for the
                // update (the update zeroes the counter when it has finished
                // the block); new blocks take item numbers in the partition
                // with one atomic per wavefront.
                const bool rsv = has && slot != kNoSlot;
                if (has) runs = L.scnt[h];
                if (rsv) {
                    roff = atomicAdd(&L.nrec, runs);            // disjoint ranges; their order does not matter
                    bc = atomicAdd(own.blk_count + slot, (1ull << 32) | runs);
                }
                const bool first = rsv && bc == 0;
                const unsigned long long fm = __ballot(first);
                if (fm) {
                    unsigned int ib = 0;
                    if (lane == 0) ib = atomicAdd(&fc->part[part].items, (unsigned int)__popcll(fm));
                    ib = read_lane0(ib);
                    if (first) {
                        const unsigned int k = ib + (unsigned int)__popcll(fm & below);
                        if (k < own.item_part_cap)
                            own.items[(size_t)part * own.item_part_cap + k] = slot;
                        else                                 // beyond the partition's share (rare)
                            own.items_spill[atomicAdd(&fc->items_spill, 1u)] = slot;
                    }
                }
            }
        }
        if (!own.build_items) continue;                      // the ray-parallel update needs nothing more
        if (d0 == 0 && tid == 0) L.r0 = r0;
        __syncthreads();
        if (has) {
            const unsigned long long rr = L.r0;
            const unsigned int seg = (unsigned int)(rr >> 32) + d;
            const unsigned int rec = (unsigned int)rr + roff;
            Segment* segs = own.segs + (size_t)part * own.seg_part_cap;
            Segment sg;
            sg.slot = kNoSlot;                               // void unless the key's runs are recorded
            sg.rec_base = 0;
            sg.block_off = 0;
            sg.seg_pos = 0;
            unsigned int rbase;
            if (slot == kNoSlot) {
                rbase = kNoKeyBase;                          // the full table refused the key: its kept visits are lost
            } else if (seg < own.seg_part_cap && (unsigned long long)rec + runs <= own.rec_part_cap &&
                       (unsigned int)(bc >> 32) <= kSegPosMask && ((unsigned int)bc & ~kSegOverflow) + runs <= kSegPosMask) {
                sg.slot = slot;
                sg.rec_base = part * own.rec_part_cap + rec;
                sg.block_off = (unsigned int)bc & ~kSegOverflow;
                sg.seg_pos = (unsigned int)(bc >> 32) | (frame << kSegFrameShift);
                rbase = sg.rec_base;
            } else {                                         // out of space (or a block's lists out of range):
                                                             // the update rescans the block
                atomicOr(own.blk_count + slot, (unsigned long long)kSegOverflow);
                rbase = kNoBase;
            }
            if (seg < own.seg_part_cap) segs[seg] = sg;      // the placing pass reads every reserved segment
            L.scnt[h] = rbase;                               // the key's runs are counted: keep its base instead
        }
    }
    __syncthreads();
    if (own.build_items) {
        // every lane: the records of its runs
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            if (!S.pend[q]) continue;
            const unsigned int b = L.scnt[hr[q] & (kSetCap - 1)];
            const unsigned long long code = L.scode[q][tid];     // w2 | (cells | kept << 8) << 32
            if (b == kNoKeyBase) {
                atomicAdd(L.cnt + 5, (unsigned int)(code >> 40));   // rare: its kept cells counted at once
            } else if (b != kNoBase) {
                RunRecord r;
                r.depth = depth;
                r.w1 = run_w1(colour_dirs, (unsigned int)(code >> 32) & 255u);
                r.w2 = (unsigned int)code;
                own.recs[b + (hr[q] >> kSetBits)] = r;
            }
        }
        __syncthreads();
    }
    // empty the set for the next filing (which starts after a barrier)
    for (unsigned int d = (unsigned int)tid; d < nu; d += kThreads) {
        const unsigned int h = L.sslot[d];
        L.skey[h] = kEmptyKey;
        L.scnt[h] = 0;
    }
    if (tid == 0) {
        L.nuniq = 0;
        L.nrun = 0;
        L.nrec = 0;
    }
}

__device__ __forceinline__ void cut_and_file(unsigned int kp, unsigned int yp, unsigned int zp, unsigned int cp,
                                             int n, int itc, int x, int y, int z, int s0, int s1, int s2, AllocLds& L,
                                             unsigned int& rnd, unsigned int part, ConstRef<VolumeArgs> vref,
                                             ConstRef<OwnerArgs> oref, unsigned int depth_bits, unsigned int colour_dirs,
                                             unsigned int frame, unsigned int& n_upd) {
    // planes in walk order, bit j = the chunk's cell j: every plane was
    // shifted once per iteration (itc of them); the lane walked n cells and
    // the bits after them are not read
    const unsigned int shp = (unsigned int)(32 - itc) & 31u;
    const unsigned int kf = itc ? __builtin_bitreverse32(kp) >> shp : 0u;
    const unsigned int yf = itc ? __builtin_bitreverse32(yp) >> shp : 0u;
    const unsigned int zf = itc ? __builtin_bitreverse32(zp) >> shp : 0u;
    const unsigned int cf = itc ? __builtin_bitreverse32(cp) >> shp : 0u;
    // cut into runs: a run ends at a cell whose step leaves the block, at
    // its kMaxRunCells-th cell, or at the lane's last cell of the chunk; up
    // to kSlots runs per lane between filings (workgroup-wide: every thread
    // takes part in each)
    for (int j0 = 0; workgroup_any(j0 < n, L, rnd);) {
        RunSlots S;
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            S.key[q] = 0;
            S.code[q] = 0;
            S.pend[q] = false;
        }
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            if (!__any(j0 < n)) break;
            if (j0 < n) {
                const unsigned int rest = cf >> j0;
                const unsigned int tz = rest ? (unsigned int)__builtin_ctz(rest) : 32u;
                const unsigned int e = min(min(tz, (unsigned int)(n - 1 - j0)),   // steps inside the run
                                           (unsigned int)(kMaxRunCells - 1));
                const unsigned int len = e + 1;                                 // its cells
                const unsigned int kept = __popc(__builtin_amdgcn_ubfe(kf, j0, len));
                const unsigned int ys = __builtin_amdgcn_ubfe(yf, j0, e);
                const unsigned int zs = __builtin_amdgcn_ubfe(zf, j0, e);
                S.key[q] = block_key(x, y, z);
                // the record's w2, with the cell count and the kept cells above it
                S.code[q] = (unsigned long long)run_w2((unsigned int)voxel_in_block(x, y, z), ys, zs) |
                            ((unsigned long long)(len | (kept << 8)) << 32);
                S.pend[q] = kept > 0;
                n_upd += kept;
                // the next run's first cell: the run's steps and the one after it
                const int cy = __popc(__builtin_amdgcn_ubfe(yf, j0, len));
                const int cz = __popc(__builtin_amdgcn_ubfe(zf, j0, len));
                x += __mul24(s0, (int)len - cy - cz);
                y += __mul24(s1, cy);
                z += __mul24(s2, cz);
                j0 += (int)len;
            }
        }
        file_runs(S, L, part, vref, oref, depth_bits, colour_dirs, frame);
    }
}

// kReproject: the reprojection reading of the occlusion test (see
// hidden_in_image) on top of the band test.
template <bool kReproject>
__global__ __launch_bounds__(kThreads, 7) void k_allocate(BatchArgs B, VolumeArgs vol, OwnerArgs own) {
    __shared__ AllocLds L;
    const int fi = blockIdx.x / B.tile_grid;                 // frame of this workgroup
    // The frame and the volume's and the update's arguments are read with
    // scalar loads where they are used: the walk's masks fill the scalar
    // registers, and values held through it would be spilled.
    const ConstRef<FrameArgs> fr = frame_ref(B, fi);
    const ConstRef<VolumeArgs> vref = const_ref(&vol);
    const ConstRef<OwnerArgs> oref = const_ref(&own);
    const FrameArgs f = load_ref(fr);                                // (the set-up's fields)
    if (blockIdx.x == 0 && own.build_items) {
        // clear the next frame's counters (their last users finished before
        // this kernel started)
        unsigned long long* next = reinterpret_cast<unsigned long long*>(own.fc + (own.parity ^ 1));
        for (int i = threadIdx.x; i < (int)(sizeof(FrameCounters) / 8); i += kThreads) next[i] = 0;
    }
    int tu, tv;
    if (!workgroup_tile(f, blockIdx.x - fi * B.tile_grid, tu, tv)) return;
    if (threadIdx.x < kProbeBins) L.hist[threadIdx.x] = 0;
    if (threadIdx.x < 6) L.cnt[threadIdx.x] = 0;
    if (threadIdx.x < 3) L.votes[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        L.pmax = 0;
        L.nuniq = 0;
        L.nrun = 0;
        L.nrec = 0;
    }
    for (int i = threadIdx.x; i < kSetCap; i += kThreads) {
        L.skey[i] = kEmptyKey;
        L.scnt[i] = 0;
    }
    // the ray slopes of the tile's 16 columns and 16 rows (the same division
    // every pixel of a column or row would do)
    if (threadIdx.x < kTile)
        L.xn[threadIdx.x] = ((float)(tu + (int)threadIdx.x) - f.cx) / f.fx;
    else if (threadIdx.x < 2 * kTile)
        L.yn[threadIdx.x - kTile] = ((float)(tv + (int)threadIdx.x - kTile) - f.cy) / f.fy;
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    int u, v;
    thread_pixel(tu, tv, u, v);
    const unsigned int pix = (unsigned int)v * (unsigned int)f.width + (unsigned int)u;
    float depth = 0.0f;
    const bool in_image = u < f.width && v < f.height;
    if (in_image) depth = f.depth[pix];
    unsigned int meta = 0;                    // colour | axis direction bits << 24 (a record's w1 without its length)
    const unsigned int depth_bits = __float_as_uint(depth);
    unsigned int n_upd = 0;
    // this workgroup's reservations: partitions in turn as if the call's
    // frames were laid end to end by their tile counts (numbering by launch
    // index instead, every frame would start at a multiple of 8 workgroups
    // and the first tiles of many small frames would all fill the same few)
    const unsigned int wg = blockIdx.x - (unsigned int)fi * (unsigned int)B.tile_grid;
    const unsigned int part = ((unsigned int)fi * (unsigned int)f.n_tiles + wg) % kParts;
    const int max_visits = f.max_visits;
    const float vs = vol.vs, trunc = vol.trunc;

    // Walk state in registers, per axis: the index of the next cell boundary
    // the walk will cross and the step (both as floats holding integers,
    // exactly), the boundary's parameter, the start and reciprocal of the
    // direction (in voxel units), and the offset from the boundary index to
    // the current cell's centre (k + 1/2 is b - 1/2 stepping up, b + 1/2
    // stepping down or still: exactly, for any cell a key can hold).
    int s0, s1, s2;
    float b0, b1, b2, f0, f1, f2, h0, h1, h2, tm0, tm1, tm2, g0, g1, g2, i0, i1, i2;
    // Lane flags are kept as wavefront lane masks (bit k: lane k) in scalar
    // registers; `lane_on` turns a mask into the lane's own condition.
    unsigned long long alive;                 // lanes whose walk goes on
    auto load_walk = [&](const BandWalk& w, bool valid) __attribute__((always_inline)) {
        // (a lane that is not valid never walks: its values go unused)
        alive = __builtin_amdgcn_ballot_w64(valid);
        s0 = w.s0; s1 = w.s1; s2 = w.s2;
        f0 = (float)s0; f1 = (float)s1; f2 = (float)s2;
        b0 = (float)(w.k0 + (s0 > 0)); b1 = (float)(w.k1 + (s1 > 0)); b2 = (float)(w.k2 + (s2 > 0));
        h0 = s0 > 0 ? -0.5f : 0.5f; h1 = s1 > 0 ? -0.5f : 0.5f; h2 = s2 > 0 ? -0.5f : 0.5f;
        tm0 = w.tm0; tm1 = w.tm1; tm2 = w.tm2;
        // an axis that does not move: start -inf and reciprocal +inf, so
        // that (b - g) i, recomputed every step, stays +inf
        g0 = s0 != 0 ? w.gA0 : -__builtin_inff();
        g1 = s1 != 0 ? w.gA1 : -__builtin_inff();
        g2 = s2 != 0 ? w.gA2 : -__builtin_inff();
        i0 = s0 != 0 ? w.inv0 : __builtin_inff();
        i1 = s1 != 0 ? w.inv1 : __builtin_inff();
        i2 = s2 != 0 ? w.inv2 : __builtin_inff();
    };
    // One step of the walk (every lane; a finished walk does not move).  The
    // stepped axis is the one whose boundary comes first (ties: x, then y);
    // its next boundary moves on by one cell, and every axis's crossing
    // parameter is then (b - g) i of its next boundary b (the same value as
    // before for an axis that did not step).  The masks of the lanes that
    // stepped, and of those that stepped along y and along z; bc the
    // boundary crossed.
    struct Step {
        unsigned long long more, e0, e1, a1, a2;
        float bc;
    };
    auto step = [&]() __attribute__((always_inline)) {
        Step st;
        const float tmin = fminf(fminf(tm0, tm1), tm2);
        st.more = alive & __builtin_amdgcn_ballot_w64(tmin <= 1.0f);
        st.e0 = __builtin_amdgcn_ballot_w64(tm0 == tmin);
        st.e1 = __builtin_amdgcn_ballot_w64(tm1 == tmin);
        const unsigned long long a0 = st.more & st.e0;
        st.a1 = st.more & ~st.e0 & st.e1;
        st.a2 = st.more & ~st.e0 & ~st.e1;
        const bool e0 = lane_on(st.e0), e1 = lane_on(st.e1);
        st.bc = pick3(e0, e1, b0, b1, b2);
        b0 = lane_on(a0) ? b0 + f0 : b0;
        b1 = lane_on(st.a1) ? b1 + f1 : b1;
        b2 = lane_on(st.a2) ? b2 + f2 : b2;
        tm0 = (b0 - g0) * i0;
        tm1 = (b1 - g1) * i1;
        tm2 = (b2 - g2) * i2;
        alive = st.more;
        return st;
    };
    const float dd = depth;
    const Projection proj = projection(f);
    const DepthAxis ax_all = depth_axis(f);  // (the reprojection walk tests every cell: held)
    auto test_sdf = [&](const DepthAxis& ax, float& sdf) __attribute__((always_inline)) {   // the centre test of the walk's current cell
        return kReproject ? centre_test_reproject_at(b0 + h0, b1 + h1, b2 + h2, dd, ax, proj, vs, trunc, sdf)
                          : centre_test_at(b0 + h0, b1 + h1, b2 + h2, dd, ax, vs, trunc, sdf);
    };
    auto test = [&]() __attribute__((always_inline)) {
        float sdf;
        return test_sdf(kReproject ? ax_all : depth_axis(load_ref(reload(fr))), sdf);   // (band walk: rare, loaded here)
    };
    // Stepped sdf (band test alone).  A step moves the centre by one voxel
    // along one axis, which changes d - zc by the pose's depth-axis entry
    // for that axis times vs.  From the exact value at a chunk's first cell
    // the walk carries sa, that value less the steps' changes in float.  The
    // band decision taken on sa is the exact test's wherever |sa| is further
    // than m from trunc, m a bound on |exact - sa| (below); lanes inside that
    // margin take the exact test.  Bound, with u = 2^-24, n <= 31 steps
    // since the first cell and r = max(1, |R entries of the depth axis|):
    // the exact test's own rounding error at a cell is at most
    // 6.001 u (r (sum_k |X_k| + sum_k |t_k|) + d) (X: the centre in world
    // units), and sum_k |X_k| grows by at most n vs, so the errors at the
    // first cell and the current one add up to at most
    // 12.01 u (r (sum |X| + sum |t| + 16 vs) + d) with X at the first cell;
    // the steps add at most u r vs each (the rounded R vs) and u |sa| each
    // (the subtraction; |sa| <= |sdf0| + 32 r vs), i.e.
    // 31 u |sdf0| + 1023 u r vs in all.
    // m = 2^-20 (r (sum |X| + sum |t| + 80 vs) + d + 2 |sdf0|) covers the sum
    // with room for the rounding of m itself, and 2^-22 trunc covers that
    // of trunc -+ m.
    const float t_abs = (fabsf(ax_all.t0) + fabsf(ax_all.t1)) + fabsf(ax_all.t2);
    const float r_max = fmaxf(fmaxf(fabsf(ax_all.r2), fabsf(ax_all.r5)), fmaxf(fabsf(ax_all.r8), 1.0f));

    // The walk goes in chunks of up to kChunkCells cells.  All lanes start
    // together, so a lane's cell index within the chunk is the (uniform)
    // iteration count; each iteration shifts one bit into four per-lane
    // planes: the cell was kept, the step after it moved along y, along z,
    // left the block.  Every lane runs the step (the stepped axis is chosen
    // by selects, not branches); a finished walk neither moves nor shifts its
    // kept plane, and its step bits stay zero.  After the chunk the planes
    // are cut into runs (one per block the chunk's part of the walk crosses)
    // and filed.  A walk longer than a chunk has its run at the chunk
    // boundary split in two records of the same block: the update adds both.
    int x, y, z;                              // the chunk's first cell
    unsigned int kp, yp, zp, cp;              // its planes
    unsigned int nc;                          // cells this lane walked in the chunk
    auto walk_chunk = [&](int done, const DepthAxis& ax) __attribute__((always_inline)) {
        x = (int)(b0 + h0 - 0.5f);            // the current cell (exact: integers and halves)
        y = (int)(b1 + h1 - 0.5f);
        z = (int)(b2 + h2 - 0.5f);
        float sa = 0.f, lo = 0.f, hi = 0.f, dl0 = 0.f, dl1 = 0.f, dl2 = 0.f;
        float sdf0;
        unsigned long long keep = __builtin_amdgcn_ballot_w64(test_sdf(ax, sdf0));   // the exact test at the chunk's first cell
        if constexpr (!kReproject) {
            sa = sdf0;
            dl0 = f0 * ax.r2 * vs;            // f (R vs), exact: f is -1, 0 or 1
            dl1 = f1 * ax.r5 * vs;            // (and rounding is symmetric)
            dl2 = f2 * ax.r8 * vs;
            // (opaque: the compiler would otherwise select f R and multiply
            // by vs in every step)
            asm volatile("" : "+v"(dl0), "+v"(dl1), "+v"(dl2));
            const float xs = (fabsf((b0 + h0) * vs) + fabsf((b1 + h1) * vs)) + fabsf((b2 + h2) * vs);
            const float m = 0x1p-20f * ((r_max * ((xs + t_abs) + 80.0f * vs) + fabsf(dd)) + 2.0f * fabsf(sdf0)) +
                            0x1p-22f * trunc;
            lo = trunc - m;
            hi = trunc + m;
        }
        kp = yp = zp = cp = nc = 0u;
        // the safety bound on cells per walk limits the chunk (uniform)
        const int lim = __builtin_amdgcn_readfirstlane(min(kChunkCells, max_visits - done));
        int itc = 0;                          // iterations of this chunk (uniform)
        for (; itc < lim; ++itc) {
            if (!alive) break;
            nc = count_in(nc, alive);         // a lane still walking is at its cell itc
            kp = shift_in(kp, keep);
            const Step st = step();
            yp = shift_in(yp, st.a1);
            zp = shift_in(zp, st.a2);
            // the step leaves the block iff the boundary it crosses is a block face
            const unsigned long long cr =
                st.more & __builtin_amdgcn_ballot_w64(__builtin_amdgcn_fractf(st.bc * 0.125f) == 0.0f);
            cp = shift_in(cp, cr);
            if constexpr (kReproject) {
                keep = __builtin_amdgcn_ballot_w64(test());
            } else {
                sa = sa - pick3(lane_on(st.e0), lane_on(st.e1), dl0, dl1, dl2);
                const float as = fabsf(sa);
                keep = __builtin_amdgcn_ballot_w64(as <= lo);
                const unsigned long long unsure = st.more & ~keep & __builtin_amdgcn_ballot_w64(as <= hi);
                if (unsure) {                 // rare: some lane is within the margin
                    const unsigned long long ex = __builtin_amdgcn_ballot_w64(test());
                    keep = (keep & ~unsure) | (ex & unsure);
                }
            }
        }
        // A walk still going after max_visits cells is cut there (counted).
        // Its last iteration took one more step; that step's bits sit after
        // the lane's last cell and no run reads them.
        if (done + lim >= max_visits) {
            const unsigned int cut = (unsigned int)__popcll(alive);
            if (cut && lane == 0) atomicAdd(L.cnt + 4, cut);
            alive = 0;
        }
        return itc;
    };
    // The workgroup goes through the chunks together (its filings are
    // collective); a wavefront whose walks have all ended skips the walk.
    bool wave_on = true;
    unsigned int rnd = 0;                     // workgroup_any's count (uniform)
    for (int done = 0;; done += kChunkCells) {
        int itc = 0;
        kp = yp = zp = cp = nc = 0u;
        x = y = z = 0;
        if (wave_on) {
            // the walk's state for this chunk: set up from the pixel, then the
            // first done steps replayed (the empty asm keeps the compiler from
            // hoisting the set-up out of the loop and holding its results)
            float dr = depth;
            float xr = L.xn[(wave & 1) * 8 + (lane & 7)], yr = L.yn[(wave >> 1) * 8 + (lane >> 3)];
            asm volatile("" : "+v"(dr), "+v"(xr), "+v"(yr));
            BandWalk w;                           // (a pixel outside the image has depth 0: invalid)
            const FrameArgs fc = load_ref(reload(fr));
            const VolumeArgs vc = load_ref(reload(vref));
            const int cls = setup_walk(w, dr, xr, yr, fc, vc.trunc, vc.inv_vs);
            load_walk(w, cls == kValid);
            if (done == 0) {
                // point classes, counted once
                const unsigned int c_valid = (unsigned int)__popcll(__ballot(cls == kValid));
                const unsigned int c_near = (unsigned int)__popcll(__ballot(cls == kNear));
                const unsigned int c_oor = (unsigned int)__popcll(__ballot(cls == kOutside));
                if (lane == 0) {
                    if (c_valid) atomicAdd(L.cnt + 0, c_valid);
                    if (c_near) atomicAdd(L.cnt + 1, c_near);
                    if (c_oor) atomicAdd(L.cnt + 2, c_oor);
                }
                // what the update needs of this point besides the run codes:
                // colour (when the frame has it) and the directions of the
                // stepping axes (the frame of the batch goes with the segments)
                if (cls == kValid) {
                    if (load_ref(reload(oref)).build_items && fc.rgb) {
                        unsigned int px = pix;       // (opaque: the address is formed here, not held from the start)
                        asm volatile("" : "+v"(px));
                        const uint8_t* c = fc.rgb + 3 * (size_t)px;
                        meta = (unsigned int)c[0] | ((unsigned int)c[1] << 8) | ((unsigned int)c[2] << 16);
                    }
                    meta |= (w.s0 < 0 ? 1u << 24 : 0u) | (w.s1 < 0 ? 1u << 25 : 0u) | (w.s2 < 0 ? 1u << 26 : 0u);
                }
            }
            for (int i = 0; i < done; ++i) step();
            itc = walk_chunk(done, depth_axis(fc));
        }
        wave_on = alive != 0;
        cut_and_file(kp, yp, zp, cp, (int)nc, itc, x, y, z, (meta >> 24) & 1u ? -1 : 1, (meta >> 25) & 1u ? -1 : 1,
                     (meta >> 26) & 1u ? -1 : 1, L, rnd, part, vref, oref, depth_bits, meta, (unsigned int)fi, n_upd);
        if (!workgroup_any(wave_on, L, rnd)) break;
    }

    const unsigned int c_upd = wave_sum(n_upd);
    if (lane == 0 && c_upd) atomicAdd(L.cnt + 3, c_upd);
    __syncthreads();
    flush_hist(L.hist, &L.pmax, vol.counters, kHistAlloc);
    if (threadIdx.x < 6 && L.cnt[threadIdx.x]) {
        const int word = threadIdx.x == 0 ? kPointsValid
                       : threadIdx.x == 1 ? kNearSkipped
                       : threadIdx.x == 2 ? kOutOfRange
                       : threadIdx.x == 3 ? kVoxelUpdates
                       : threadIdx.x == 4 ? kWalkGuard
                                          : kUpdateMisses;
        atomicAdd(replica(vol.counters) + word, (unsigned long long)L.cnt[threadIdx.x]);
    }
}

// ---------------------------------------------------------------------------
// grouping the call's run records by block.  k_place_items gives every
// touched block a descriptor and a contiguous range of the block-ordered
// segment list (one atomic per 256 blocks); k_place_segments puts each
// segment's (first record, runs before it) at its position in that range.
// The records themselves stay where allocate wrote them.
// ---------------------------------------------------------------------------
// prefix over the partitions' counts (+ the spill list): pre[p] = first
// global index of partition p, pre[kParts + 1] = total
__device__ void partition_prefix(const unsigned int* counts, unsigned int cap, unsigned int spill, unsigned int* pre) {
    if (threadIdx.x == 0) {
        unsigned int acc = 0;
        for (int p = 0; p < kParts; ++p) {
            pre[p] = acc;
            acc += min(counts[p], cap);
        }
        pre[kParts] = acc;
        pre[kParts + 1] = acc + spill;
    }
    __syncthreads();
}

__device__ __forceinline__ int find_partition(const unsigned int* pre, unsigned int i) {
    int a = 0, b = kParts;                   // largest p with pre[p] <= i (p = kParts: spill)
    while (a < b) {
        const int m = (a + b + 1) >> 1;
        if (pre[m] <= i) a = m; else b = m - 1;
    }
    return a;
}

__global__ __launch_bounds__(kThreads) void k_place_items(VolumeArgs vol, OwnerArgs own) {
    __shared__ unsigned int s_cnt[kParts];
    __shared__ unsigned int s_pre[kParts + 2];
    __shared__ unsigned int s_wave[kWaves];
    __shared__ unsigned int s_base;
    __shared__ unsigned int s_runs;
    __shared__ unsigned int s_front[kWaves], s_back[kWaves];
    __shared__ unsigned int s_fbase, s_bbase;
    FrameCounters& fc = own.fc[own.parity];
    if (threadIdx.x < kParts) s_cnt[threadIdx.x] = fc.part[threadIdx.x].items;
    if (threadIdx.x < 64) {                  // the call's runs (records reserved in all partitions)
        const unsigned int r = (unsigned int)fc.part[threadIdx.x].segrec;
        const unsigned int t = wave_sum(r);
        if (threadIdx.x == 0) s_runs = t;
    }
    static_assert(kParts == 64, "one wavefront sums the partitions' records");
    __syncthreads();
    partition_prefix(s_cnt, own.item_part_cap, fc.items_spill, s_pre);
    const unsigned int n = s_pre[kParts + 1];
    const unsigned int mean_runs = s_runs / max(n, 1u);
    // runs per work unit: a block with more is split (the call's runs over
    // unit_target units, so the units of all split blocks fit the list)
    const unsigned int unit_runs = max(kMinUnitRuns, (s_runs + own.unit_target - 1) / max(own.unit_target, 1u));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        fc.items_total = n;
        fc.unit_runs = unit_runs;
        // this call's allocate has claimed its pool indices: the next call's
        // fresh blocks start where they end
        own.fc[own.parity ^ 1].pool_start = min(vol.counters[kBlockCounter], vol.capacity);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (unsigned int b = blockIdx.x * kThreads; b < n; b += gridDim.x * kThreads) {
        const unsigned int i = b + tid;
        unsigned int slot = 0, rc = 0, nseg = 0, cnt = 0;
        if (i < n) {
            const int p = find_partition(s_pre, i);
            slot = p < kParts ? own.items[(size_t)p * own.item_part_cap + (i - s_pre[p])]
                              : own.items_spill[i - s_pre[kParts]];
            const unsigned long long bc = own.blk_count[slot];
            rc = (unsigned int)bc;
            nseg = (unsigned int)(bc >> 32);
            cnt = (rc & kSegOverflow) ? 0u : nseg;
        }
        // The item's number, the order the update takes blocks in: blocks
        // with more runs than the call's mean from the front, the others
        // from the back, so that no long block starts when the rest of the
        // work is nearly done.  One add per workgroup and class, with the
        // segment placement's.
        const bool big = i < n && (rc & ~kSegOverflow) > mean_runs;
        const bool small = i < n && !big;
        const unsigned long long mb = __ballot(big), ms = __ballot(small);
        if (lane == 0) {
            s_front[wave] = (unsigned int)__popcll(mb);
            s_back[wave] = (unsigned int)__popcll(ms);
        }
        unsigned int x = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_wave[wave] = x;
        __syncthreads();
        if (tid == 0) {
            unsigned int acc = 0, af = 0, ab = 0;
            for (int k = 0; k < kWaves; ++k) {
                const unsigned int t = s_wave[k], tf = s_front[k], tb = s_back[k];
                s_wave[k] = acc;
                s_front[k] = af;
                s_back[k] = ab;
                acc += t;
                af += tf;
                ab += tb;
            }
            s_base = (unsigned int)atomicAdd(&fc.placed, (unsigned long long)acc);
            s_fbase = af ? atomicAdd(&fc.front, af) : 0u;
            s_bbase = ab ? atomicAdd(&fc.back, ab) : 0u;
        }
        __syncthreads();
        const unsigned long long below = (1ull << lane) - 1ull;
        const unsigned int j = big ? s_fbase + s_front[wave] + (unsigned int)__popcll(mb & below)
                                   : n - 1u - (s_bbase + s_back[wave] + (unsigned int)__popcll(ms & below));
        if (i < n) {
            const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(vol.table + slot);
            ItemDesc d;
            d.key = e.x;
            d.idx = (unsigned int)e.y;
            d.rec_count = rc;
            d.seg_first = s_base + s_wave[wave] + x - cnt;
            d.seg_count = cnt;
            d.slot = slot;
            d.units = 1;
            if (!(rc & kSegOverflow) && rc > unit_runs) {
                // chunks 1.. of the block go to the list of extra units
                // (their number over all blocks is at most the call's runs
                // over unit_runs <= unit_target <= kMaxUnits)
                const unsigned int extra = (rc + unit_runs - 1) / unit_runs - 1;
                const unsigned int u0 = atomicAdd(&fc.n_extra, extra);
                if (u0 + extra <= kMaxUnits) {
                    for (unsigned int c = 1; c <= extra; ++c) own.units[u0 + c - 1] = make_uint2(j, c);
                    d.units = extra + 1;
                } else {                     // (cannot happen, see above) entries marked void
                    for (unsigned int c = 1; c <= extra && u0 + c - 1 < kMaxUnits; ++c)
                        own.units[u0 + c - 1] = make_uint2(0xFFFFFFFFu, 0u);
                }
            }
            own.desc[j] = d;
            own.seg_first_of[slot] = (rc & kSegOverflow) ? kNoSlot : d.seg_first;
            if (rc & kSegOverflow) own.rescan[atomicAdd(&fc.n_rescan, 1u)] = j;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void k_place_segments(VolumeArgs vol, OwnerArgs own) {
    __shared__ unsigned int s_cnt[kParts];
    __shared__ unsigned int s_pre[kParts + 2];
    FrameCounters& fc = own.fc[own.parity];
    if (threadIdx.x < kParts) s_cnt[threadIdx.x] = (unsigned int)(fc.part[threadIdx.x].segrec >> 32);
    __syncthreads();
    partition_prefix(s_cnt, own.seg_part_cap, 0, s_pre);
    const unsigned int n = s_pre[kParts];
    for (unsigned int j = blockIdx.x * kThreads + threadIdx.x; j < n; j += gridDim.x * kThreads) {
        const int p = find_partition(s_pre, j);
        const Segment sg = own.segs[(size_t)p * own.seg_part_cap + (j - s_pre[p])];
        if (sg.slot == kNoSlot) continue;                       // refused for lack of space
        const unsigned int first = own.seg_first_of[sg.slot];
        if (first == kNoSlot) continue;                         // the block is rescanned
        own.seg_list[first + (sg.seg_pos & kSegPosMask)] =
            make_uint2(sg.rec_base, sg.block_off | (sg.seg_pos & ~kSegPosMask));   // (the frame rides along)
    }
}

// Drop a frame's records without updating (an allocate that no update
// followed): clear the per-block run counts it left.
__global__ __launch_bounds__(kThreads) void k_discard_items(VolumeArgs vol, OwnerArgs own) {
    __shared__ unsigned int s_cnt[kParts];
    __shared__ unsigned int s_pre[kParts + 2];
    FrameCounters& fc = own.fc[own.parity];
    if (threadIdx.x < kParts) s_cnt[threadIdx.x] = fc.part[threadIdx.x].items;
    __syncthreads();
    partition_prefix(s_cnt, own.item_part_cap, fc.items_spill, s_pre);
    const unsigned int n = s_pre[kParts + 1];
    // this call's allocate cleared its successor's counters, pool_start
    // included, and no k_place_items will run for it: record here where the
    // next call's fresh pool blocks start
    if (blockIdx.x == 0 && threadIdx.x == 0)
        own.fc[own.parity ^ 1].pool_start = min(vol.counters[kBlockCounter], vol.capacity);
    for (unsigned int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const int p = find_partition(s_pre, i);
        const unsigned int slot = p < kParts ? own.items[(size_t)p * own.item_part_cap + (i - s_pre[p])]
                                             : own.items_spill[i - s_pre[kParts]];
        own.blk_count[slot] = 0;
    }
}

// ---------------------------------------------------------------------------
// owner update: one workgroup per touched block at a time, blocks handed out
// through one work counter per XCD.  The block's run records are staged in
// LDS with coalesced loads and sorted by length, so the lanes of a wavefront
// replay runs of about the same length together; each run's cells follow
// from its recorded first cell and step planes (the walk's arithmetic is not
// repeated) and get the centre test.  Kept voxels add into LDS (integer
// words, see below), and the block's touched voxels are then read, added to
// and written with plain coalesced loads and stores: the block has no other
// writer in this call.  Blocks whose runs did not fit the record buffers are
// left to k_update_rescan.
// ---------------------------------------------------------------------------
// The chunk's sums per voxel live in two 64-bit LDS words added with integer
// atomics (LDS float atomics issue far slower than integer ones on this
// chip).  A run adds at most once to each voxel, so a chunk of at most
// kChunkRuns = 8191 runs keeps every per-voxel count below 2^13:
//   tw   normalised signed distance in units of 2^-24, rounded to nearest,
//        plus 2^25 (the distance times 1/trunc may pass +-1 by an ulp, so each
//        term lies in (0, 2^26), the sum below 2^39) in bits 0-50,
//        | count << 51
//   rgb  R | G << 21 | B << 42 (each sum at most 255 * 8191 < 2^21)
// so no field carries into the next.  The signed-distance sum is recovered
// exactly from the two fields; rounding each term to the nearest 2^-24 (the
// float's own spacing for terms of magnitude 1/2 to 1) moves a mean by at
// most 2^-25.
constexpr unsigned int kChunkRuns = 8191;
constexpr int kSegWindow = 256;                      // segments of a block held in LDS at once
constexpr int kUpdateThreads = 256;                  // workgroup of the owner update
constexpr int kRunsPerThread = 2;                    // runs each thread stages (2: 22.3 KB of LDS and
                                                     // 72 VGPRs, 7 workgroups per CU)
constexpr int kSubRuns = kUpdateThreads * kRunsPerThread;   // runs staged in LDS at a time
constexpr int kLengths = 32;                         // run lengths a record can state (5 bits)
constexpr unsigned int kNoRank = 0xFFFFFFFFu;
constexpr float kTsdfScale = 16777216.0f;            // 2^24
constexpr float kTsdfUnit = 1.0f / 16777216.0f;
constexpr int kCountShift = 51;                      // the count's place in the tw word
constexpr unsigned long long kTsdfMask = (1ull << kCountShift) - 1ull;
constexpr int kRescanThreads = 128;

// Voxel j's sums sit at sum_slot(j): one spare word after every 16, so that
// voxels 32 apart (neighbouring rays' cells four rows apart, say) no longer
// fall on the same LDS banks.
constexpr int kSumSlots = kBlockVoxels + kBlockVoxels / 16;
__device__ __forceinline__ int sum_slot(int j) { return j + (j >> 4); }

struct OwnerLds {
    unsigned long long tw[kSumSlots];
    unsigned long long rgb[kSumSlots];
};

// Add the chunk's sums to the pool block and clear them for the next chunk.
// fresh: the pool block still holds the zeros the pool was cleared to, so the
// sums are written without reading it first (0 + x is x exactly).
__device__ __forceinline__ void flush_owner(OwnerLds& L, const VolumeArgs& vol, size_t base, bool fresh) {
    for (int j = threadIdx.x; j < kBlockVoxels; j += kUpdateThreads) {
        const unsigned long long tw = L.tw[sum_slot(j)];
        const unsigned int cnt = (unsigned int)(tw >> kCountShift);
        if (!cnt) continue;
        const unsigned long long c = L.rgb[sum_slot(j)];
        // sum of the signed distances, in units of 2^-24 (the 2^25 offsets removed)
        const long long tq = (long long)(tw & kTsdfMask) - ((long long)cnt << 25);
        const float ts = (float)tq * kTsdfUnit;
        L.tw[sum_slot(j)] = 0;
        L.rgb[sum_slot(j)] = 0;
        const size_t off = base + j;
        float t0 = 0.0f, w0 = 0.0f, r0 = 0.0f, g0 = 0.0f, b0 = 0.0f;
        if (!fresh) {
            t0 = vol.tsdf[off];
            w0 = vol.weight[off];
            r0 = vol.r[off];
            g0 = vol.g[off];
            b0 = vol.b[off];
        }
        vol.tsdf[off] = t0 + ts;
        vol.weight[off] = w0 + (float)cnt;
        vol.r[off] = r0 + (float)((unsigned int)c & 0x1FFFFFu) * kInv255;
        vol.g[off] = g0 + (float)((unsigned int)(c >> 21) & 0x1FFFFFu) * kInv255;
        vol.b[off] = b0 + (float)((unsigned int)(c >> 42) & 0x1FFFFFu) * kInv255;
    }
}

// A block refused a pool index: its kept cells (counted, not stored), and
// the sums cleared for the next pass.
__device__ __forceinline__ unsigned int count_and_clear(OwnerLds& L) {
    unsigned int n = 0;
    for (int j = threadIdx.x; j < kBlockVoxels; j += kUpdateThreads) {
        n += (unsigned int)(L.tw[sum_slot(j)] >> kCountShift);
        L.tw[sum_slot(j)] = 0;
        L.rgb[sum_slot(j)] = 0;
    }
    return n;
}

// The same for one work unit of a split block: other workgroups add to the
// same voxels, so the sums go in with no-return float atomics (weights stay
// exact: integer-valued floats far below 2^24).
__device__ __forceinline__ void flush_atomic(OwnerLds& L, const VolumeArgs& vol, size_t base) {
    for (int j = threadIdx.x; j < kBlockVoxels; j += kUpdateThreads) {
        const unsigned long long tw = L.tw[sum_slot(j)];
        const unsigned int cnt = (unsigned int)(tw >> kCountShift);
        if (!cnt) continue;
        const unsigned long long c = L.rgb[sum_slot(j)];
        const long long tq = (long long)(tw & kTsdfMask) - ((long long)cnt << 25);
        L.tw[sum_slot(j)] = 0;
        L.rgb[sum_slot(j)] = 0;
        const size_t off = base + j;
        unsafeAtomicAdd(vol.tsdf + off, (float)tq * kTsdfUnit);
        unsafeAtomicAdd(vol.weight + off, (float)cnt);
        unsafeAtomicAdd(vol.r + off, (float)((unsigned int)c & 0x1FFFFFu) * kInv255);
        unsafeAtomicAdd(vol.g + off, (float)((unsigned int)(c >> 21) & 0x1FFFFFu) * kInv255);
        unsafeAtomicAdd(vol.b + off, (float)((unsigned int)(c >> 42) & 0x1FFFFFu) * kInv255);
    }
}

// A run as the update stages it in LDS: its record and its segment's frame.
struct __align__(16) StagedRun {
    unsigned int depth;
    unsigned int w1;
    unsigned int w2;
    unsigned int frame;
};

// kReproject: the reprojection reading of the occlusion test (as in k_allocate).
template <bool kReproject>
__global__ __launch_bounds__(kUpdateThreads, kReproject ? 5 : 7) void k_update_owner(BatchArgs B, VolumeArgs vol, OwnerArgs own) {
    __shared__ OwnerLds L;
    __shared__ DepthAxis s_axis[kMaxBatch];                 // per-record frame lookups from LDS
    __shared__ Projection s_proj[kMaxBatch];
    __shared__ unsigned int s_item[2];                      // alternates: read k while k + 1 is written
    // the window's segments: first record, and runs before it | frame << kSegFrameShift
    __shared__ uint2 s_seg[kSegWindow + 1];
    __shared__ StagedRun s_run[kSubRuns];                   // staged runs, sorted by length
    __shared__ unsigned int s_hist[kLengths];               // staged runs of each length
    __shared__ unsigned int s_hbase[kLengths];              // first place of each length in the order
    const int tid = threadIdx.x;
    if (tid < kLengths) s_hist[tid] = 0;
    if (tid < B.n) {
        s_axis[tid] = depth_axis(*frame_ptr(B, tid));
        if (kReproject) s_proj[tid] = projection(*frame_ptr(B, tid));
    }
    for (int j = tid; j < kBlockVoxels; j += kUpdateThreads) {
        L.tw[sum_slot(j)] = 0;
        L.rgb[sum_slot(j)] = 0;
    }
    FrameCounters& fc = own.fc[own.parity];
    const unsigned int n_items = fc.items_total;
    const unsigned long long fresh_from = fc.pool_start;
    // sdf / trunc in units of 2^-24: (sdf * (1/trunc)) * 2^24 rounds exactly
    // as sdf * ((1/trunc) * 2^24) (scaling by a power of two is exact)
    const float tsdf_scale = vol.inv_trunc * kTsdfScale;
    const unsigned int xcd = blockIdx.x % kXcds;
    unsigned int* fetch = fc.fetch + xcd * kFetchStride;
    unsigned int misses = 0;
    // work: the extra units of split blocks first, then every block (a split
    // block's own entry does its first unit)
    const unsigned int n_extra = min(fc.n_extra, kMaxUnits);
    const unsigned int unit_runs = fc.unit_runs;

    for (unsigned int k = 0;; ++k) {
        if (tid == 0) s_item[k & 1] = xcd + kXcds * atomicAdd(fetch, 1u);
        __syncthreads();                                     // also: LDS sums clear, frames loaded
        const unsigned int wi = s_item[k & 1];
        if (wi >= n_extra + n_items) break;
        unsigned int it = wi - n_extra, chunk = 0;
        if (wi < n_extra) {
            const uint2 u = own.units[wi];
            it = u.x;
            chunk = u.y;
            if (it >= n_items) continue;                     // a void entry
        }
        const ItemDesc d = own.desc[it];
        if (d.rec_count & kSegOverflow) continue;            // rescanned (and its count cleared) later
        if (chunk >= d.units) continue;
        if (chunk == 0 && tid == 0) own.blk_count[d.slot] = 0;
        const bool split = d.units > 1;
        // this unit's runs of the block, in block order
        const unsigned int r_lo = split ? chunk * unit_runs : 0u;
        const unsigned int r_hi = split ? min(d.rec_count, r_lo + unit_runs) : d.rec_count;
        const bool store = d.idx < vol.capacity;             // else refused a pool index: count, not store
        bool fresh = !split && d.idx >= fresh_from;          // no update has written the block yet
        int bx, by, bz;
        unpack_key(d.key, bx, by, bz);
        const int lo0 = bx * 8, lo1 = by * 8, lo2 = bz * 8;
        const size_t base = (size_t)d.idx * kBlockVoxels;
        // the block's segments, a window at a time: segment i holds runs
        // [off(i), off(i + 1)) of the block (off: the low kSegFrameShift bits
        // of s_seg[i].y), stored from s_seg[i].x on
        for (unsigned int w0 = 0; w0 < d.seg_count; w0 += kSegWindow) {
            const unsigned int wn = min(d.seg_count - w0, (unsigned int)kSegWindow);
            for (unsigned int i = tid; i <= wn; i += kUpdateThreads) {
                if (i < wn) {
                    s_seg[i] = own.seg_list[d.seg_first + w0 + i];
                } else {
                    s_seg[i] = make_uint2(0u, w0 + wn < d.seg_count ? own.seg_list[d.seg_first + w0 + wn].y & kSegPosMask
                                                                    : d.rec_count);
                }
            }
            __syncthreads();
            const unsigned int wr0 = max(s_seg[0].y & kSegPosMask, r_lo), wr1 = min(s_seg[wn].y, r_hi);
            const bool past = s_seg[wn].y >= r_hi;           // (uniform) no later window holds this unit's runs
            for (unsigned int c0 = wr0; c0 < wr1; c0 += kChunkRuns) {
                const unsigned int c1 = min(wr1, c0 + kChunkRuns);
                // The chunk's runs go through LDS kSubRuns at a time: each
                // thread loads kRunsPerThread neighbouring runs (a wavefront's
                // loads cover whole cache lines of records), the staged runs
                // are sorted by length (a counting sort over LDS), and each
                // thread then replays every kUpdateThreads-th run in that
                // order.  The lanes of a wavefront so replay runs of nearly
                // the same length in step, and few idle while the longest
                // finishes.
                for (unsigned int b0 = c0; b0 < c1; b0 += kSubRuns) {
                    const unsigned int nb = min(c1 - b0, (unsigned int)kSubRuns);
                    const unsigned int p0 = (unsigned int)tid * kRunsPerThread;
                    StagedRun rec[kRunsPerThread];
                    unsigned int rank[kRunsPerThread];
#pragma unroll
                    for (int i = 0; i < kRunsPerThread; ++i) rank[i] = kNoRank;
                    if (p0 < nb) {
                        unsigned int r = b0 + p0;
                        unsigned int lo = 0, hi = wn - 1;    // last segment starting at or before r
                        while (lo < hi) {
                            const unsigned int m = (lo + hi + 1) >> 1;
                            if ((s_seg[m].y & kSegPosMask) <= r) lo = m; else hi = m - 1;
                        }
                        unsigned int si = lo;
                        uint2 cur = s_seg[si];                // segment si, and where the next one starts
                        unsigned int next = s_seg[si + 1].y & kSegPosMask;
#pragma unroll
                        for (int i = 0; i < kRunsPerThread; ++i) {
                            if (p0 + i < nb) {
                                while (r >= next) {           // (the sentinel s_seg[wn] = wr1 > r ends it)
                                    cur = s_seg[++si];
                                    next = s_seg[si + 1].y & kSegPosMask;
                                }
                                const RunRecord hr = own.recs[cur.x + (r - (cur.y & kSegPosMask))];
                                rec[i].depth = hr.depth;
                                rec[i].w1 = hr.w1;
                                rec[i].w2 = hr.w2;
                                rec[i].frame = cur.y >> kSegFrameShift;
                                ++r;
                            }
                        }
#pragma unroll
                        for (int i = 0; i < kRunsPerThread; ++i) {
                            if (p0 + i < nb) rank[i] = atomicAdd(s_hist + run_cells(rec[i].w1) - 1, 1u);
                        }
                    }
                    __syncthreads();
                    if (tid < 64) {                          // each length's first place in the order
                        const unsigned int h = tid < kLengths ? s_hist[tid] : 0u;
                        const unsigned int incl = wave_inclusive_sum(h);
                        if (tid < kLengths) s_hbase[tid] = incl - h;
                    }
                    __syncthreads();
                    if (tid < kLengths) s_hist[tid] = 0;     // for the next sub-batch
#pragma unroll
                    for (int i = 0; i < kRunsPerThread; ++i)
                        if (rank[i] != kNoRank)
                            s_run[s_hbase[run_cells(rec[i].w1) - 1] + rank[i]] = rec[i];
                    __syncthreads();
                    for (unsigned int p = (unsigned int)tid; p < nb; p += kUpdateThreads) {
                        const StagedRun rr = s_run[p];
                        const float dep = __uint_as_float(rr.depth);
                        const int rf = (int)rr.frame;
                        const DepthAxis ax = s_axis[__umul24(rr.frame, 1u)];    // (a 24-bit index: a cheap multiply)
                        const unsigned long long c = (unsigned long long)(rr.w1 & 0xFFu) |
                                                     ((unsigned long long)((rr.w1 >> 8) & 0xFFu) << 21) |
                                                     ((unsigned long long)((rr.w1 >> 16) & 0xFFu) << 42);
                        // the axis directions, as voxel-index steps (a step
                        // along x, y or z adds d0, d0 + dy or d0 + dz) and
                        // as floats
                        const bool n0 = (rr.w1 >> 24) & 1u, n1 = (rr.w1 >> 25) & 1u, n2 = (rr.w1 >> 26) & 1u;
                        const int d0 = n0 ? -1 : 1;
                        const int dy = (n1 ? -8 : 8) - d0, dz = (n2 ? -64 : 64) - d0;
                        const float f0 = n0 ? -1.0f : 1.0f, f1 = n1 ? -1.0f : 1.0f, f2 = n2 ? -1.0f : 1.0f;
                        const int e = run_entry(rr.w2), cells = run_cells(rr.w1);
                        // the cell's centre in voxels, k + 1/2 per axis (exact:
                        // integers and halves), and its voxel within the block
                        // (a run stays in its block)
                        float x0 = (float)(lo0 + (e & 7)) + 0.5f;
                        float x1 = (float)(lo1 + ((e >> 3) & 7)) + 0.5f;
                        float x2 = (float)(lo2 + (e >> 6)) + 0.5f;
                        int j = e;
                        const unsigned int ys = run_ysteps(rr.w2), zs = run_zsteps(rr.w2);
                        // q counts the cells every active lane has done (the
                        // same in all of them, a scalar)
                        for (int q = 0; q < cells; ++q) {
                            float sdf;
                            if (kReproject ? centre_test_reproject_at(x0, x1, x2, dep, ax, s_proj[rf], vol.vs, vol.trunc, sdf)
                                           : centre_test_at(x0, x1, x2, dep, ax, vol.vs, vol.trunc, sdf)) {
                                const unsigned int tq = (unsigned int)(__float2int_rn(sdf * tsdf_scale) + (1 << 25));
                                atomicAdd(L.tw + sum_slot(j), (1ull << kCountShift) + tq);
                                atomicAdd(L.rgb + sum_slot(j), c);
                            }
                            // the step after cell q: bit q of the planes (after
                            // the run's last cell both are 0, an x step whose
                            // cell is never used).  The coordinates move by
                            // exactly 0 or +-1, so the fused multiply-add rounds
                            // nothing.
                            const int by = (int)__builtin_amdgcn_ubfe(ys, (unsigned int)q, 1u);
                            const int bz = (int)__builtin_amdgcn_ubfe(zs, (unsigned int)q, 1u);
                            const int bx = 1 - by - bz;
                            x0 = __builtin_fmaf((float)bx, f0, x0);
                            x1 = __builtin_fmaf((float)by, f1, x1);
                            x2 = __builtin_fmaf((float)bz, f2, x2);
                            j += d0 + by * dy + bz * dz;
                        }
                    }
                    __syncthreads();                         // s_run is rewritten next
                }
                __syncthreads();
                if (!store)
                    misses += count_and_clear(L);            // refused a pool index: its kept cells are lost
                else if (split)
                    flush_atomic(L, vol, base);
                else
                    flush_owner(L, vol, base, fresh);
                fresh = false;                               // a later pass adds to what this one wrote
                __syncthreads();
            }
            __syncthreads();                                 // the window may be reloaded
            if (past) break;
        }
    }
    const unsigned int c_miss = wave_sum(misses);
    if ((tid & 63) == 0 && c_miss) atomicAdd(replica(vol.counters) + kUpdateMisses, (unsigned long long)c_miss);
}

// ---------------------------------------------------------------------------
// rescan of the blocks whose runs did not fit the record buffers: in every
// frame of the batch, every pixel of the rectangle the block's band can be
// seen through replays its walk through the block.  Counts can exceed the
// packed word's range here, so weight and colour sums are kept as separate
// 32-bit integer halves.
// ---------------------------------------------------------------------------
struct RescanLds {
    float tsdf[kBlockVoxels];
    unsigned long long wr[kBlockVoxels];          // weight | R sum << 32
    unsigned long long gb[kBlockVoxels];          // G sum | B sum << 32
};

__global__ __launch_bounds__(kRescanThreads) void k_update_rescan(BatchArgs B, VolumeArgs vol, OwnerArgs own) {
    __shared__ RescanLds L;
    FrameCounters& fc = own.fc[own.parity];
    const unsigned int n = fc.n_rescan;
    unsigned int misses = 0, done = 0;
    for (unsigned int q = blockIdx.x; q < n; q += gridDim.x) {
        const ItemDesc d = own.desc[own.rescan[q]];
        int bx, by, bz;
        unpack_key(d.key, bx, by, bz);
        for (int j = threadIdx.x; j < kBlockVoxels; j += kRescanThreads) {
            L.tsdf[j] = 0.0f;
            L.wr[j] = 0;
            L.gb[j] = 0;
        }
        __syncthreads();
        unsigned int n_kept = 0;
        const int lo0 = bx * 8, lo1 = by * 8, lo2 = bz * 8;
        for (int fi = 0; fi < B.n; ++fi) {
            const FrameArgs f = batch_frame(B, fi);
            const Projection pr = projection(f);
            const DepthAxis fax = depth_axis(f);
            const PixelRect rc = block_rect(bx, by, bz, f, vol.vs);
            if (rc.u0 > rc.u1 || rc.v0 > rc.v1) continue;
            const int rw = rc.u1 - rc.u0 + 1;
            const long long area = (long long)rw * (rc.v1 - rc.v0 + 1);
            const float zlo = rc.zmin - vol.vs, zhi = rc.zmax + vol.vs;
            for (long long p = threadIdx.x; p < area; p += kRescanThreads) {
                const int u = rc.u0 + (int)(p % rw);
                const int v = rc.v0 + (int)(p / rw);
                const size_t pix = (size_t)v * f.width + u;
                const float dep = f.depth[pix];
                if (!(dep - vol.trunc <= zhi && dep + vol.trunc >= zlo)) continue;   // band cannot reach the block
                BandWalk w;
                if (setup_walk(w, dep, u, v, f, vol.trunc, vol.inv_vs) != kValid) continue;
                if (w.span_hi0 < lo0 - 1 || w.span_lo0 > lo0 + 8 || w.span_hi1 < lo1 - 1 || w.span_lo1 > lo1 + 8 ||
                    w.span_hi2 < lo2 - 1 || w.span_lo2 > lo2 + 8)
                    continue;                                                     // cell span misses the block
                const unsigned long long c_wr = 1ull | ((unsigned long long)f.rgb[3 * pix + 0] << 32);
                const unsigned long long c_gb =
                    (unsigned long long)f.rgb[3 * pix + 1] | ((unsigned long long)f.rgb[3 * pix + 2] << 32);
                bool inside = false;
                for (int visits = 0;;) {
                    if ((unsigned)(w.k0 - lo0) < 8u && (unsigned)(w.k1 - lo1) < 8u && (unsigned)(w.k2 - lo2) < 8u) {
                        inside = true;
                        float sdf;
                        if (vol.reproject
                                ? centre_test_reproject(w.k0, w.k1, w.k2, w.d, fax, pr, vol.vs, vol.trunc, sdf)
                                : centre_test(w, f, vol.vs, vol.trunc, sdf)) {
                            const int j = voxel_in_block(w.k0, w.k1, w.k2);
                            atomicAdd(L.tsdf + j, sdf * vol.inv_trunc);
                            atomicAdd(L.wr + j, c_wr);
                            atomicAdd(L.gb + j, c_gb);
                            ++n_kept;
                        }
                    } else if (inside) {
                        break;                                                // a walk crosses a block once
                    }
                    if (++visits >= f.max_visits || !advance(w)) break;
                }
            }
        }
        __syncthreads();
        if (d.idx < vol.capacity) {
            const size_t base = (size_t)d.idx * kBlockVoxels;
            for (int j = threadIdx.x; j < kBlockVoxels; j += kRescanThreads) {
                const unsigned long long wr = L.wr[j];
                const unsigned int cnt = (unsigned int)wr;
                if (!cnt) continue;
                const unsigned long long gb = L.gb[j];
                const size_t off = base + j;
                const float t0 = vol.tsdf[off], w0 = vol.weight[off], r0 = vol.r[off], g0 = vol.g[off],
                            b0 = vol.b[off];
                vol.tsdf[off] = t0 + L.tsdf[j];
                vol.weight[off] = w0 + (float)cnt;
                vol.r[off] = r0 + (float)(unsigned int)(wr >> 32) * kInv255;
                vol.g[off] = g0 + (float)(unsigned int)gb * kInv255;
                vol.b[off] = b0 + (float)(unsigned int)(gb >> 32) * kInv255;
            }
        } else {
            misses += n_kept;               // block refused a pool index: counted, not stored
        }
        if (threadIdx.x == 0) {
            own.blk_count[d.slot] = 0;
            ++done;
        }
        __syncthreads();
    }
    const unsigned int c_miss = wave_sum(misses);
    if ((threadIdx.x & 63) == 0 && c_miss) atomicAdd(replica(vol.counters) + kUpdateMisses, (unsigned long long)c_miss);
    if (threadIdx.x == 0 && done) atomicAdd(replica(vol.counters) + kFallbackBlocks, (unsigned long long)done);
}

// ---------------------------------------------------------------------------
// ray-parallel update: walk, test, look the block up once per block run of
// the ray, add with five no-return f32 atomics into the SoA pool.
// ---------------------------------------------------------------------------
// Per-wavefront staging of block-index lookups: a small LDS hash map from
// block key to pool index.  A lane entering a block takes the index from the
// map; when the key is not there yet, the lanes that need it in the same
// step enter it with an LDS compare-exchange, the one that entered it looks
// it up in the table, and after a wavefront fence every one of them reads
// the index.  A wavefront's rays cross a few blocks, so most runs need no
// table probe at all.  A full map (more than kLookupCap distinct keys in a
// wavefront) sends the lane to the table directly.
constexpr int kLookupCap = 64;

struct LookupLds {
    unsigned long long key[kWaves][kLookupCap];
    unsigned int idx[kWaves][kLookupCap];
};

__device__ __forceinline__ unsigned int staged_lookup(LookupLds& M, int wave, const VolumeArgs& vol,
                                                      unsigned long long key, unsigned int* s_hist,
                                                      unsigned int* s_pmax) {
    unsigned long long* mk = M.key[wave];
    unsigned int* mi = M.idx[wave];
    unsigned int h = set_slot(key) & (kLookupCap - 1), n = 0;
    bool won = false, found = false;
    for (; n < (unsigned int)kLookupCap; ++n) {
        const unsigned long long prev = atomicCAS(&mk[h], kEmptyKey, key);
        if (prev == kEmptyKey) {
            won = true;
            break;
        }
        if (prev == key) {
            found = true;
            break;
        }
        h = (h + 1) & (kLookupCap - 1);
    }
    unsigned int idx = kNoIndex;
    if (won || !found) {                     // the entering lane, or a full map: the table
        unsigned int probes;
        idx = lookup_key(vol, key, probes);
        hist_add(s_hist, s_pmax, probes);
        if (won) mi[h] = idx;
    }
    // the entries written in this step are visible to the whole wavefront
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (found) idx = mi[h];
    return idx;
}

__global__ __launch_bounds__(kThreads) void k_update_rays(BatchArgs B, VolumeArgs vol) {
    const int fi = blockIdx.x / B.tile_grid;
    const FrameArgs f = batch_frame(B, fi);
    __shared__ unsigned int s_hist[kProbeBins];
    __shared__ unsigned int s_pmax;
    __shared__ unsigned int s_miss;
    __shared__ LookupLds M;
    int tu, tv;
    if (!workgroup_tile(f, blockIdx.x - fi * B.tile_grid, tu, tv)) return;
    if (threadIdx.x < kProbeBins) s_hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        s_pmax = 0;
        s_miss = 0;
    }
    for (int i = threadIdx.x; i < kWaves * kLookupCap; i += kThreads) (&M.key[0][0])[i] = kEmptyKey;
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int u, v;
    thread_pixel(tu, tv, u, v);
    BandWalk w;
    int cls = kInvalid;
    float cr = 0.f, cg = 0.f, cb = 0.f;
    if (u < f.width && v < f.height) {
        const size_t pix = (size_t)v * f.width + u;
        cls = setup_walk(w, f.depth[pix], u, v, f, vol.trunc, vol.inv_vs);
        if (cls == kValid) {
            cr = (float)f.rgb[3 * pix + 0] * kInv255;
            cg = (float)f.rgb[3 * pix + 1] * kInv255;
            cb = (float)f.rgb[3 * pix + 2] * kInv255;
        }
    }
    unsigned int n_miss = 0;
    const Projection pr = projection(f);
    const DepthAxis fax = depth_axis(f);
    if (cls == kValid) {
        unsigned long long cur = kEmptyKey;
        unsigned int idx = kNoIndex;
        int visits = 0;
        for (;;) {
            float sdf;
            if (vol.reproject ? centre_test_reproject(w.k0, w.k1, w.k2, w.d, fax, pr, vol.vs, vol.trunc, sdf)
                              : centre_test(w, f, vol.vs, vol.trunc, sdf)) {
                const unsigned long long key = block_key(w.k0, w.k1, w.k2);
                if (key != cur) {
                    idx = staged_lookup(M, wave, vol, key, s_hist, &s_pmax);
                    cur = key;
                }
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
            bool crossed;
            int axis;
            if (++visits >= f.max_visits || !advance_select(w, crossed, axis)) break;
        }
    }
    const unsigned int c_miss = wave_sum(n_miss);
    if ((threadIdx.x & 63) == 0 && c_miss) atomicAdd(&s_miss, c_miss);
    __syncthreads();
    flush_hist(s_hist, &s_pmax, vol.counters, kHistUpdate);
    if (threadIdx.x == 0 && s_miss) atomicAdd(replica(vol.counters) + kUpdateMisses, (unsigned long long)s_miss);
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

// Zero the first `capacity` pool blocks of all five arrays or, with
// use_counter, only min(block counter, capacity) blocks (the used part).
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

__global__ __launch_bounds__(kThreads) void k_zero_words(unsigned int* a, unsigned long long n) {
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (unsigned long long)gridDim.x * blockDim.x)
        a[i] = 0;
}

// Launch parameters of up to kArgFrames frames, copied word by word from the
// kernel arguments into the device frame table (frames beyond the kernel
// arguments of a call's own kernels).
struct FrameGroup {
    FrameArgs f[kArgFrames];
};

__global__ __launch_bounds__(kThreads) void k_store_frames(FrameGroup g, FrameArgs* table, int n) {
    constexpr int kWords = (int)(sizeof(FrameArgs) / 4);
    const unsigned int* src = reinterpret_cast<const unsigned int*>(g.f);
    unsigned int* dst = reinterpret_cast<unsigned int*>(table);
    for (int i = threadIdx.x; i < n * kWords; i += blockDim.x) dst[i] = src[i];
}

// The call's fresh-block start: pool indices from the block counter's
// current value on have never been written by an update.
__global__ void k_set_pool_start(FrameCounters* fc, const unsigned long long* counters,
                                 unsigned long long capacity) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const unsigned long long used = counters[kBlockCounter];
        fc->pool_start = used < capacity ? used : capacity;
    }
}

__global__ __launch_bounds__(kThreads) void k_zero_counters(unsigned long long* counters) {
    for (int i = threadIdx.x; i < kReplicas * kCounterWords; i += blockDim.x) counters[i] = 0;
}

__global__ __launch_bounds__(kThreads) void k_export_coords(const Entry* table, unsigned long long n_entries,
                                                             unsigned long long n_blocks, int* coords) {
    for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n_entries;
         i += (unsigned long long)gridDim.x * blockDim.x) {
        const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(table + i);
        const unsigned int idx = (unsigned int)e.y;
        if (e.x == kEmptyKey || idx >= n_blocks) continue;
        int bx, by, bz;
        unpack_key(e.x, bx, by, bz);
        coords[3 * (size_t)idx + 0] = bx;
        coords[3 * (size_t)idx + 1] = by;
        coords[3 * (size_t)idx + 2] = bz;
    }
}

unsigned int grid_for(unsigned long long n) {
    unsigned long long g = (n + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > 8192) g = 8192;
    return (unsigned int)g;
}

bool launched() { return hipGetLastError() == hipSuccess; }

}  // namespace

// ---------------------------------------------------------------------------
// launch wrappers
// ---------------------------------------------------------------------------
int tile_grid(const FrameArgs& f) { return f.tiles_per_xcd * kXcds; }

const char* kernel_name(int id) {
    static const char* const names[kKernelIds] = {"k_allocate",      "k_place_items", "k_place_segments",
                                                  "k_update_owner",  "k_update_rescan", "k_discard_items",
                                                  "k_update_rays"};
    return id >= 0 && id < kKernelIds ? names[id] : "unknown";
}

#define TSDF_TIMED_LAUNCH(timer, id, kernel, grid, block, stream, ...)            \
    do {                                                                          \
        if (timer) (timer)->mark((timer)->ctx, (id), 0, (stream));                \
        hipLaunchKernelGGL(kernel, (grid), (block), 0, (stream), __VA_ARGS__);    \
        if (timer) (timer)->mark((timer)->ctx, (id), 1, (stream));                \
    } while (0)

bool launch_allocate(const BatchArgs& b, const VolumeArgs& v, const OwnerArgs& o, hipStream_t s,
                     const LaunchTimer* t) {
    if (v.reproject)
        TSDF_TIMED_LAUNCH(t, kKAllocate, k_allocate<true>, dim3(b.n * b.tile_grid), dim3(kThreads), s, b, v, o);
    else
        TSDF_TIMED_LAUNCH(t, kKAllocate, k_allocate<false>, dim3(b.n * b.tile_grid), dim3(kThreads), s, b, v, o);
    return launched();
}

bool launch_update_owner(const BatchArgs& b, const VolumeArgs& v, const OwnerArgs& o, int grid, hipStream_t s,
                         const LaunchTimer* t) {
    TSDF_TIMED_LAUNCH(t, kKPlaceItems, k_place_items, dim3(256), dim3(kThreads), s, v, o);
    TSDF_TIMED_LAUNCH(t, kKPlaceSegments, k_place_segments, dim3(1024), dim3(kThreads), s, v, o);
    if (v.reproject)
        TSDF_TIMED_LAUNCH(t, kKUpdateOwner, k_update_owner<true>, dim3(grid), dim3(kUpdateThreads), s, b, v, o);
    else
        TSDF_TIMED_LAUNCH(t, kKUpdateOwner, k_update_owner<false>, dim3(grid), dim3(kUpdateThreads), s, b, v, o);
    TSDF_TIMED_LAUNCH(t, kKUpdateRescan, k_update_rescan, dim3(256), dim3(kRescanThreads), s, b, v, o);
    return launched();
}

int owner_grid(bool reproject) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const void* k = reproject ? reinterpret_cast<const void*>(k_update_owner<true>)
                              : reinterpret_cast<const void*>(k_update_owner<false>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kUpdateThreads, 0) != hipSuccess) return 0;
    return std::max(1, cus) * std::max(1, per_cu);
}

bool launch_discard(const VolumeArgs& v, const OwnerArgs& o, hipStream_t s, const LaunchTimer* t) {
    TSDF_TIMED_LAUNCH(t, kKDiscardItems, k_discard_items, dim3(64), dim3(kThreads), s, v, o);
    return launched();
}

bool launch_update_rays(const BatchArgs& b, const VolumeArgs& v, hipStream_t s, const LaunchTimer* t) {
    TSDF_TIMED_LAUNCH(t, kKUpdateRays, k_update_rays, dim3(b.n * b.tile_grid), dim3(kThreads), s, b, v);
    return launched();
}

bool launch_init(const VolumeArgs& v, unsigned long long table_entries, bool whole_pool, const OwnerArgs* own,
                 hipStream_t s) {
    if (own) {
        hipLaunchKernelGGL(k_zero_words, dim3(grid_for(2 * table_entries)), dim3(kThreads), 0, s,
                           reinterpret_cast<unsigned int*>(own->blk_count), 2 * table_entries);
        hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(kThreads), 0, s, reinterpret_cast<unsigned int*>(own->fc),
                           (unsigned long long)(2 * sizeof(FrameCounters) / 4));
    }
    const unsigned long long cap = v.capacity;
    hipLaunchKernelGGL(k_zero_pool, dim3(grid_for(cap * (kBlockVoxels / 4))), dim3(kThreads), 0, s,
                       (float4*)v.tsdf, (float4*)v.weight, (float4*)v.r, (float4*)v.g, (float4*)v.b,
                       (const unsigned long long*)v.counters, cap, whole_pool ? 0 : 1);
    hipLaunchKernelGGL(k_fill_table, dim3(grid_for(table_entries)), dim3(kThreads), 0, s, (uint4*)v.table,
                       table_entries);
    hipLaunchKernelGGL(k_zero_counters, dim3(1), dim3(kThreads), 0, s, v.counters);
    return launched();
}

bool launch_store_frames(const FrameArgs* frames, int n, FrameArgs* table, hipStream_t s) {
    for (int i = 0; i < n; i += kArgFrames) {
        FrameGroup g;
        const int k = std::min(kArgFrames, n - i);
        for (int j = 0; j < k; ++j) g.f[j] = frames[i + j];
        hipLaunchKernelGGL(k_store_frames, dim3(1), dim3(kThreads), 0, s, g, table + i, k);
    }
    return launched();
}

bool launch_fresh_call(const VolumeArgs& v, const OwnerArgs& o, unsigned long long table_entries, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(kThreads), 0, s, reinterpret_cast<unsigned int*>(o.fc),
                       (unsigned long long)(2 * sizeof(FrameCounters) / 4));
    hipLaunchKernelGGL(k_zero_words, dim3(grid_for(2 * table_entries)), dim3(kThreads), 0, s,
                       reinterpret_cast<unsigned int*>(o.blk_count), 2 * table_entries);
    hipLaunchKernelGGL(k_set_pool_start, dim3(1), dim3(64), 0, s, o.fc + o.parity,
                       (const unsigned long long*)v.counters, v.capacity);
    return launched();
}

bool launch_hand_back(const VolumeArgs& v, FrameCounters* next, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(kThreads), 0, s, reinterpret_cast<unsigned int*>(next),
                       (unsigned long long)(sizeof(FrameCounters) / 4));
    hipLaunchKernelGGL(k_set_pool_start, dim3(1), dim3(64), 0, s, next, (const unsigned long long*)v.counters,
                       v.capacity);
    return launched();
}

bool launch_export_coords(const VolumeArgs& v, unsigned long long table_entries, unsigned long long n_blocks,
                          int* coords, hipStream_t s) {
    hipLaunchKernelGGL(k_export_coords, dim3(grid_for(table_entries)), dim3(kThreads), 0, s, v.table, table_entries,
                       n_blocks, coords);
    return launched();
}

}  // namespace tsdf
