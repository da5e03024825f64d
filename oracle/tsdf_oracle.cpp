/*
 * tsdf_oracle.cpp -- reference ("oracle") integrator for hash-blocked TSDF
 * fusion.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it to check and time the HIP library.
 * The HIP library never links, loads or calls it, and the two share no code.
 *
 * What it computes follows "What Irregularity Costs: CUDA C++, Rust, and
 * Triton on a Hash-Blocked GPU Workload", section 3 (method):
 *   - the volume is cut into blocks of 8^3 voxels; each voxel keeps five
 *     float quantities: truncated signed distance, weight, R, G, B;
 *   - integration walks the truncation band of every depth point, and each
 *     voxel it touches that passes the occlusion test gets one contribution;
 *   - the pool stores weighted SUMS, not running means (sums commute); the
 *     mean is sum / weight, recovered only for checking;
 *   - allocation and update apply the same occlusion test, so a block exists
 *     if and only if one of its voxels received a contribution (bounded by
 *     the pool capacity; blocks beyond it are refused and counted);
 *   - the signed distance is taken at the voxel centre (section 4 reports the
 *     half-voxel bias of evaluating it at the ray sample instead).
 * Where the pages leave a step open (the band walk, the occlusion test, the
 * units, the f32 rounding order), this file follows the written float
 * contract that the HIP kernels also follow, independently:
 *
 *   C0  inv_vs = 1/vs (f32).  All arithmetic f32, round-to-nearest, no FMA
 *       contraction, correctly rounded division, evaluated as written.
 *   C1  depth d: finite and > 0, else the pixel is invalid.  d <= trunc:
 *       "near" (the band would reach the camera plane), skipped and counted.
 *   C2  xn = (u - cx) / fx, yn = (v - cy) / fy   (pixel indices, OpenCV)
 *   C3  band segment in camera coordinates from z0 = d - trunc to
 *       z1 = d + trunc along the pixel ray: a = z0 (xn, yn, 1), b = z1 (..)
 *   C4  to world, then to voxel units:  g = (((R_i0 a0 + R_i1 a1) + R_i2 a2)
 *       + t_i) * inv_vs.  A point whose segment end has |g_i| > 2^23 - 8 on
 *       any axis (or NaN) is out of the key range: skipped and counted.
 *   C5  voxel walk: Amanatides-Woo traversal of the half-open unit cells the
 *       segment gA->gB passes through, parameter s in [0, 1]; next-boundary
 *       parameters tmax_i = (boundary - gA_i) / dir_i computed as
 *       (boundary - gA_i) * (1/dir_i); an axis with |dir_i| <= 1e-30 never
 *       steps; the smallest tmax steps, ties to the lowest axis (x, y, z);
 *       stop once the smallest tmax exceeds 1.
 *   C6  every visited cell k: centre c_i = (k_i + 0.5) vs, camera depth of
 *       the centre zc = (R_02 (c0 - t0) + R_12 (c1 - t1)) + R_22 (c2 - t2),
 *       sdf = d - zc.  Occlusion test: keep iff sdf >= -trunc (a centre more
 *       than trunc behind the observed surface is hidden) and sdf <= trunc
 *       (band).
 *   C7  a kept cell contributes tsdf = sdf / trunc, weight 1, colour
 *       channel / 255 to its voxel; block = floor(k / 8) per axis, voxel
 *       index within the block = (k0 mod 8) + 8 (k1 mod 8) + 64 (k2 mod 8).
 *   C8  (the reprojection reading of the occlusion test, ORACLE_REPROJECT):
 *       a cell that passes C6 is also hidden, and skipped, when the depth
 *       image itself shows a surface more than trunc in front of its centre
 *       along the centre's own line of sight: with q = c - t, the centre in
 *       camera coordinates is xc = (R_00 q0 + R_10 q1) + R_20 q2, yc likewise
 *       with column 1, zc as in C6; for zc > 0 it projects to
 *       uf = ((xc / zc) fx + cx) + 0.5, vf = ((yc / zc) fy + cy) + 0.5 and to
 *       the pixel (floor(uf), floor(vf)) (nearest pixel centre); if that
 *       pixel is inside the image and its depth D is finite and > 0, the
 *       cell is hidden iff zc - D > trunc.  Without such evidence (outside
 *       the image, no valid depth there, zc <= 0) it is not hidden.
 *
 * The oracle keeps blocks in a std::map keyed by block coordinate and adds
 * each contribution in double (the exact sum the f32 atomics approximate).
 * Pixels are taken in raster order, frames in call order.
 */
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <memory>
#include <set>
#include <vector>

namespace {

constexpr int kBlockEdge = 8;
constexpr int kBlockVoxels = kBlockEdge * kBlockEdge * kBlockEdge;
constexpr float kRangeLimit = 8388600.0f;      // 2^23 - 8 voxels
constexpr float kStillAxis = 1e-30f;

struct Coord {
    int32_t x, y, z;
    bool operator<(const Coord& o) const {
        if (x != o.x) return x < o.x;
        if (y != o.y) return y < o.y;
        return z < o.z;
    }
};

struct Sums {
    double tsdf[kBlockVoxels];
    double weight[kBlockVoxels];
    double r[kBlockVoxels];
    double g[kBlockVoxels];
    double b[kBlockVoxels];
};

struct Block {
    std::unique_ptr<Sums> sums;
    std::unique_ptr<uint32_t[]> voxel_frame;  // last frame + 1 per voxel (counts only)
    std::unique_ptr<uint32_t[]> voxel_call;   // last call that touched the voxel (counts only)
    uint32_t block_frame = 0;                 // last frame + 1 that touched it
    uint32_t block_call = 0;                  // last call that touched it
    uint32_t created_call = 0;                // the call that created it
};

int floor_div8(int k) {
    int q = k / kBlockEdge;
    if (k % kBlockEdge != 0 && k < 0) q -= 1;
    return q;
}

}  // namespace

extern "C" {

/* per-frame counts; all plain integers */
typedef struct {
    int64_t pixels;            /* W*H */
    int64_t points_valid;      /* depth finite, > trunc, in key range */
    int64_t near_skipped;      /* 0 < d <= trunc */
    int64_t out_of_range;      /* segment outside +-2^23 voxels */
    int64_t cells_visited;     /* cells the walks visited */
    int64_t voxel_updates;     /* kept (point, voxel) pairs: V */
    int64_t blocks_touched;    /* distinct pool blocks with a kept voxel: B_t */
    int64_t blocks_new;        /* blocks created this frame: B_n */
    int64_t voxels_touched;    /* distinct pool voxels with a kept visit: U */
    int64_t update_misses;     /* kept visits whose block was refused */
    int64_t pool_overflow_new; /* distinct keys refused this frame */
} oracle_frame_stats;

/* counts of one call: the frames integrated since the last oracle_begin_call
 * (or since creation).  A call stands for one batched launch of several
 * frames: it reads and writes each block it touches once. */
typedef struct {
    int64_t frames;            /* frames in the call */
    int64_t blocks_touched;    /* distinct pool blocks with a kept voxel in the call: B_call */
    int64_t blocks_new;        /* blocks the call created */
    int64_t voxels_fresh;      /* distinct voxels with a kept visit, in blocks the call created */
    int64_t voxels_old;        /* distinct voxels with a kept visit, in blocks created earlier */
} oracle_call_stats;

typedef struct {
    int64_t blocks;            /* blocks in the pool */
    int64_t pool_overflow;     /* distinct keys refused (pool full) */
    int64_t update_misses;
    int64_t points_valid, near_skipped, out_of_range, voxel_updates;
    int64_t frames;
} oracle_totals;

enum { ORACLE_TRACK_TOUCHED = 1, ORACLE_REPROJECT = 4 };

struct oracle_volume {
    float vs, trunc, inv_vs;
    int64_t capacity;
    int32_t flags;
    std::map<Coord, Block> blocks;
    std::set<Coord> refused;
    oracle_totals tot;
    uint32_t call = 1;         // the current call
    oracle_call_stats cs;      // its counts
};

/* C7: one kept cell k of a point with signed distance sdf and colour col. */
static void contribute(oracle_volume* o, oracle_frame_stats& s, uint32_t stamp, const int k[3],
                       float sdf, const float col[3]) {
    s.voxel_updates++;
    const Coord bc{floor_div8(k[0]), floor_div8(k[1]), floor_div8(k[2])};
    const int local = (k[0] - kBlockEdge * bc.x) + kBlockEdge * (k[1] - kBlockEdge * bc.y) +
                      kBlockEdge * kBlockEdge * (k[2] - kBlockEdge * bc.z);
    auto it = o->blocks.find(bc);
    if (it == o->blocks.end()) {
        if ((int64_t)o->blocks.size() >= o->capacity) {    // pool exhausted: refuse, count
            if (o->refused.insert(bc).second) s.pool_overflow_new++;
            s.update_misses++;
            return;
        }
        it = o->blocks.emplace(bc, Block()).first;
        s.blocks_new++;
        o->cs.blocks_new++;
        it->second.created_call = o->call;
        it->second.sums.reset(new Sums());
        std::memset(it->second.sums.get(), 0, sizeof(Sums));
        if (o->flags & ORACLE_TRACK_TOUCHED) {
            it->second.voxel_frame.reset(new uint32_t[kBlockVoxels]);
            std::memset(it->second.voxel_frame.get(), 0, sizeof(uint32_t) * kBlockVoxels);
            it->second.voxel_call.reset(new uint32_t[kBlockVoxels]);
            std::memset(it->second.voxel_call.get(), 0, sizeof(uint32_t) * kBlockVoxels);
        }
    }
    Block& blk = it->second;
    if (blk.block_frame != stamp) {
        blk.block_frame = stamp;
        s.blocks_touched++;
    }
    if (blk.block_call != o->call) {
        blk.block_call = o->call;
        o->cs.blocks_touched++;
    }
    if (blk.voxel_frame && blk.voxel_frame[local] != stamp) {
        blk.voxel_frame[local] = stamp;
        s.voxels_touched++;
    }
    if (blk.voxel_call && blk.voxel_call[local] != o->call) {
        blk.voxel_call[local] = o->call;
        if (blk.created_call == o->call)
            o->cs.voxels_fresh++;
        else
            o->cs.voxels_old++;
    }
    Sums& S = *blk.sums;
    S.tsdf[local] += (double)sdf / (double)o->trunc;
    S.weight[local] += 1.0;
    S.r[local] += (double)col[0] / 255.0;
    S.g[local] += (double)col[1] / 255.0;
    S.b[local] += (double)col[2] / 255.0;
}

/* C8: is the centre c (camera depth zc) of a cell hidden behind the surface
 * the depth image shows at its own projection? */
static bool hidden(const float* depth, int32_t W, int32_t H, float fx, float fy, float cx, float cy,
                   const float* R, const float* t, const float c[3], float zc, float trunc) {
    if (!(zc > 0.0f)) return false;
    const float q0 = c[0] - t[0], q1 = c[1] - t[1], q2 = c[2] - t[2];
    const float xc = (R[0] * q0 + R[3] * q1) + R[6] * q2;
    const float yc = (R[1] * q0 + R[4] * q1) + R[7] * q2;
    const float uf = ((xc / zc) * fx + cx) + 0.5f;
    const float vf = ((yc / zc) * fy + cy) + 0.5f;
    if (!(uf >= 0.0f && uf < (float)W && vf >= 0.0f && vf < (float)H)) return false;
    const int64_t iu = (int64_t)std::floor(uf), iv = (int64_t)std::floor(vf);
    const float D = depth[iv * W + iu];
    if (!std::isfinite(D) || !(D > 0.0f)) return false;
    return zc - D > trunc;
}

void* oracle_create(float voxel_size, float trunc, int64_t pool_capacity, int32_t flags) {
    if (!(voxel_size > 0.0f) || !(trunc > 0.0f) || pool_capacity < 0) return nullptr;
    oracle_volume* o = new oracle_volume();
    o->vs = voxel_size;
    o->trunc = trunc;
    o->inv_vs = 1.0f / voxel_size;
    o->capacity = pool_capacity;
    o->flags = flags;
    std::memset(&o->tot, 0, sizeof(o->tot));
    std::memset(&o->cs, 0, sizeof(o->cs));
    return o;
}

void oracle_destroy(void* h) { delete static_cast<oracle_volume*>(h); }

/* Start a new call: the frames integrated from here on are counted as one
 * batch by oracle_get_call_stats. */
void oracle_begin_call(void* h) {
    oracle_volume* o = static_cast<oracle_volume*>(h);
    o->call++;
    std::memset(&o->cs, 0, sizeof(o->cs));
}

void oracle_get_call_stats(void* h, oracle_call_stats* out) { *out = static_cast<oracle_volume*>(h)->cs; }

int oracle_integrate(void* h, const float* depth, const uint8_t* rgb, int32_t W, int32_t H,
                     float fx, float fy, float cx, float cy, const float* R, const float* t,
                     oracle_frame_stats* st) {
    oracle_volume* o = static_cast<oracle_volume*>(h);
    if (W < 0 || H < 0) return -1;
    oracle_frame_stats s;
    std::memset(&s, 0, sizeof(s));
    s.pixels = (int64_t)W * H;
    const uint32_t stamp = (uint32_t)o->tot.frames + 1;
    const float vs = o->vs, trunc = o->trunc, inv_vs = o->inv_vs;

    for (int32_t v = 0; v < H; ++v) {
        for (int32_t u = 0; u < W; ++u) {
            const int64_t pix = (int64_t)v * W + u;
            const float d = depth[pix];
            if (!std::isfinite(d) || !(d > 0.0f)) continue;               // C1
            if (d <= trunc) { s.near_skipped++; continue; }

            const float xn = ((float)u - cx) / fx;                         // C2
            const float yn = ((float)v - cy) / fy;
            const float z0 = d - trunc, z1 = d + trunc;                    // C3
            const float a[3] = {xn * z0, yn * z0, z0};
            const float b[3] = {xn * z1, yn * z1, z1};
            float gA[3], gB[3];
            bool in_range = true;
            for (int i = 0; i < 3; ++i) {                                  // C4
                const float Ai = ((R[3 * i + 0] * a[0] + R[3 * i + 1] * a[1]) + R[3 * i + 2] * a[2]) + t[i];
                const float Bi = ((R[3 * i + 0] * b[0] + R[3 * i + 1] * b[1]) + R[3 * i + 2] * b[2]) + t[i];
                gA[i] = Ai * inv_vs;
                gB[i] = Bi * inv_vs;
                if (!(std::fabs(gA[i]) <= kRangeLimit) || !(std::fabs(gB[i]) <= kRangeLimit)) in_range = false;
            }
            if (!in_range) { s.out_of_range++; continue; }
            s.points_valid++;

            const float col[3] = {(float)rgb[3 * pix + 0], (float)rgb[3 * pix + 1], (float)rgb[3 * pix + 2]};

            // C5: traversal set-up
            int k[3], step[3];
            float inv[3], tmax[3];
            for (int i = 0; i < 3; ++i) {
                k[i] = (int)std::floor(gA[i]);
                const float dir = gB[i] - gA[i];
                if (dir > kStillAxis) {
                    step[i] = 1;
                    inv[i] = 1.0f / dir;
                    tmax[i] = ((float)(k[i] + 1) - gA[i]) * inv[i];
                } else if (dir < -kStillAxis) {
                    step[i] = -1;
                    inv[i] = 1.0f / dir;
                    tmax[i] = ((float)k[i] - gA[i]) * inv[i];
                } else {
                    step[i] = 0;
                    inv[i] = 0.0f;
                    tmax[i] = INFINITY;
                }
            }

            for (;;) {
                s.cells_visited++;
                // C6: test the centre of cell k
                float c[3];
                for (int i = 0; i < 3; ++i) c[i] = ((float)k[i] + 0.5f) * vs;
                const float zc = (R[2] * (c[0] - t[0]) + R[5] * (c[1] - t[1])) + R[8] * (c[2] - t[2]);
                const float sdf = d - zc;
                if (sdf >= -trunc && sdf <= trunc) {
                    if (!(o->flags & ORACLE_REPROJECT) || !hidden(depth, W, H, fx, fy, cx, cy, R, t, c, zc, trunc))
                        contribute(o, s, stamp, k, sdf, col);
                }
                // C5: advance to the next cell along the segment
                int m = 0;
                if (tmax[1] < tmax[m]) m = 1;
                if (tmax[2] < tmax[m]) m = 2;
                if (!(tmax[m] <= 1.0f)) break;
                k[m] += step[m];
                const int boundary = step[m] > 0 ? k[m] + 1 : k[m];
                tmax[m] = ((float)boundary - gA[m]) * inv[m];
            }
        }
    }

    o->tot.frames++;
    o->cs.frames++;
    o->tot.blocks = (int64_t)o->blocks.size();
    o->tot.pool_overflow += s.pool_overflow_new;
    o->tot.update_misses += s.update_misses;
    o->tot.points_valid += s.points_valid;
    o->tot.near_skipped += s.near_skipped;
    o->tot.out_of_range += s.out_of_range;
    o->tot.voxel_updates += s.voxel_updates;
    if (st) *st = s;
    return 0;
}

void oracle_get_totals(void* h, oracle_totals* out) { *out = static_cast<oracle_volume*>(h)->tot; }

int64_t oracle_block_count(void* h) { return (int64_t)static_cast<oracle_volume*>(h)->blocks.size(); }

/* All block coordinates (n x 3), ascending (x, then y, then z). */
void oracle_block_coords(void* h, int32_t* coords) {
    int64_t i = 0;
    for (const auto& kv : static_cast<oracle_volume*>(h)->blocks) {
        coords[3 * i + 0] = kv.first.x;
        coords[3 * i + 1] = kv.first.y;
        coords[3 * i + 2] = kv.first.z;
        ++i;
    }
}

/* Sums of the requested blocks, 512 per block in voxel-index order.  Blocks
 * that are absent are filled with NaN.  Returns how many of the requested
 * blocks exist. */
int64_t oracle_block_sums(void* h, const int32_t* coords, int64_t n, double* tsdf, double* weight,
                          double* r, double* g, double* b) {
    oracle_volume* o = static_cast<oracle_volume*>(h);
    int64_t found = 0;
    for (int64_t i = 0; i < n; ++i) {
        auto it = o->blocks.find(Coord{coords[3 * i], coords[3 * i + 1], coords[3 * i + 2]});
        const Sums* S = (it != o->blocks.end()) ? it->second.sums.get() : nullptr;
        for (int j = 0; j < kBlockVoxels; ++j) {
            const int64_t q = i * kBlockVoxels + j;
            tsdf[q] = S ? S->tsdf[j] : NAN;
            weight[q] = S ? S->weight[j] : NAN;
            r[q] = S ? S->r[j] : NAN;
            g[q] = S ? S->g[j] : NAN;
            b[q] = S ? S->b[j] : NAN;
        }
        if (S) ++found;
    }
    return found;
}

}  // extern "C"
