// tsdf_mesh.hip -- surface extraction on gfx950: marching tetrahedra over
// the fused volume, and its host launch wrapper (tsdf_kernels.hpp).
//
// "What Irregularity Costs: CUDA C++, Rust, and Triton on a Hash-Blocked GPU
// Workload", section 3, extracts the surface once after integration by
// marching tetrahedra; section 3a gates on the extracted surface (the
// analytic sphere within a quarter voxel, distances between vertex sets).
// Conventions (the pages name the method only):
//   * samples at voxel centres ((k + 1/2) vs); a voxel is observed iff its
//     weight sum is > 0; its value is the mean TSDF, and it is inside (behind
//     the surface) iff its TSDF sum is < 0;
//   * the cell with lower corner at voxel k is cut along its main diagonal
//     into six tetrahedra, one per ordering (a, b, c) of the axes, in the
//     order xyz, xzy, yxz, yzx, zxy, zyx: corners k, k + e_a, k + e_a + e_b,
//     k + (1, 1, 1); a tetrahedron with an unobserved corner is skipped;
//   * an edge from lattice point p to p + d (d in {0,1}^3) whose ends lie on
//     opposite sides holds the vertex (p, d) at P + t (Q - P),
//     t = v_p / (v_p - v_q);
//   * triangles face from inside to outside: with s = +1 for the orderings
//     xyz, yzx, zxy and -1 otherwise, a lone inside corner i (others j < k <
//     l) gives (ij, ik, il) when the permutation (i, j, k, l) has sign s,
//     else (ij, il, ik); a lone outside corner the opposite order; two
//     inside i0 < i1 and two outside o0 < o1 give the quad (i0o0, i0o1,
//     i1o1, i1o0) when (i0, i1, o0, o1) has sign s, else (i0o0, i1o0, i1o1,
//     i0o1), cut into (V0, V1, V2) and (V0, V2, V3).
//
// Workgroups scan the table in 256-slot stretches and extract each block
// found there: the block's 8^3 voxels and the first layer of its +x, +y, +z
// neighbours (found through the hash table) are staged in LDS as 9^3 means
// with their inside / observed flags; each thread takes two cells, counts
// its triangles, the workgroup reserves their output range with one atomic,
// and each thread writes its triangles: nine floats of vertex positions and
// (optionally) twelve integers of vertex names (x, y, z, d per vertex) each.
#include <hip/hip_runtime.h>

#include "tsdf_kernels.hpp"

namespace tsdf {
namespace {

constexpr int kMeshThreads = 256;
constexpr int kSide = 9;                       // a block's 8 voxels plus one of the next block
constexpr int kLattice = kSide * kSide * kSide;
constexpr unsigned char kObserved = 1, kInside = 2;

struct MeshLds {
    float v[kLattice];                         // mean TSDF
    unsigned char flag[kLattice];              // kObserved | kInside
    unsigned int nb[8];                        // pool index of the block at offset (n & 1, n >> 1 & 1, n >> 2)
    unsigned int scan[kMeshThreads / 64];
    unsigned long long base;
};

__device__ __forceinline__ int lat(int x, int y, int z) { return x + kSide * (y + kSide * z); }

// sign of the permutation (a, b, c, d) of 0..3
__device__ __forceinline__ int perm_parity(int a, int b, int c, int d) {
    int inv = (a > b) + (a > c) + (a > d) + (b > c) + (b > d) + (c > d);
    return (inv & 1) ? -1 : 1;
}

// the tetrahedra of a cell: corner offsets of P1 and P2 (P0 = 0, P3 = (1,1,1))
// as bit masks x | y << 1 | z << 2, and their orientation signs
__constant__ int kTetA[6] = {1, 1, 2, 2, 4, 4};
__constant__ int kTetB[6] = {3, 5, 3, 6, 5, 6};
__constant__ int kTetSign[6] = {1, -1, -1, 1, 1, -1};

struct CellCorner {
    int off;           // offset bits within the cell
    int l;             // lattice index in LDS
};

// One tetrahedron's triangles: count them, or (write) emit them.
struct TriOut {
    float* pos;                        // 9 floats per triangle
    int* key;                          // 12 ints per triangle
    unsigned long long next, limit;    // next triangle index, max_triangles
};

__device__ __forceinline__ void put_vertex(const MeshLds& L, const CellCorner& p, const CellCorner& q, int gx, int gy,
                                           int gz, float vs, float* pos, int* key) {
    // p is the lower end: q - p has components 0 or 1
    const int px = gx + (p.off & 1), py = gy + ((p.off >> 1) & 1), pz = gz + ((p.off >> 2) & 1);
    const int d = q.off & ~p.off;
    const int qx = px + (d & 1), qy = py + ((d >> 1) & 1), qz = pz + ((d >> 2) & 1);
    const float vp = L.v[p.l], vq = L.v[q.l];
    const float t = vp / (vp - vq);
    const float P0 = ((float)px + 0.5f) * vs, P1 = ((float)py + 0.5f) * vs, P2 = ((float)pz + 0.5f) * vs;
    const float Q0 = ((float)qx + 0.5f) * vs, Q1 = ((float)qy + 0.5f) * vs, Q2 = ((float)qz + 0.5f) * vs;
    pos[0] = P0 + t * (Q0 - P0);
    pos[1] = P1 + t * (Q1 - P1);
    pos[2] = P2 + t * (Q2 - P2);
    if (!key) return;
    key[0] = px;
    key[1] = py;
    key[2] = pz;
    key[3] = d;
}

// Triangles of tetrahedron `tet` of the cell at LDS corner (x, y, z), global
// lattice point (gx, gy, gz).  With out == nullptr only counts.
__device__ __forceinline__ int tet_triangles(const MeshLds& L, int x, int y, int z, int gx, int gy, int gz, int tet,
                                             float vs, TriOut* out) {
    CellCorner c[4];
    const int offs[4] = {0, kTetA[tet], kTetB[tet], 7};
    int n_in = 0, mask_in = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i].off = offs[i];
        c[i].l = lat(x + (offs[i] & 1), y + ((offs[i] >> 1) & 1), z + ((offs[i] >> 2) & 1));
        const unsigned char fl = L.flag[c[i].l];
        if (!(fl & kObserved)) return 0;
        if (fl & kInside) {
            ++n_in;
            mask_in |= 1 << i;
        }
    }
    if (n_in == 0 || n_in == 4) return 0;
    const int n_tri = n_in == 2 ? 2 : 1;
    if (!out) return n_tri;
    const int s = kTetSign[tet];
    // the vertex on the edge between corners a and b (lower index = lower end)
    int va[4], vb[4];                          // up to four vertices, as corner pairs
    int tri[2][3];
    if (n_in != 2) {
        const bool lone_inside = n_in == 1;
        int lone = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (((mask_in >> i) & 1) == (lone_inside ? 1 : 0)) lone = i;
        int r[3], k = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i != lone) r[k++] = i;
        const bool same = perm_parity(lone, r[0], r[1], r[2]) * s > 0;
        // forward order (lone-r0, lone-r1, lone-r2) faces away from the lone corner
        const bool fwd = same == lone_inside;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            va[i] = min(lone, r[i]);
            vb[i] = max(lone, r[i]);
        }
        tri[0][0] = 0;
        tri[0][1] = fwd ? 1 : 2;
        tri[0][2] = fwd ? 2 : 1;
    } else {
        int in[2], ou[2], a = 0, b = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if ((mask_in >> i) & 1) in[a++] = i; else ou[b++] = i;
        }
        const bool same = perm_parity(in[0], in[1], ou[0], ou[1]) * s > 0;
        // quad in cyclic order
        const int qa[4] = {in[0], same ? in[0] : in[1], in[1], same ? in[1] : in[0]};
        const int qb[4] = {ou[0], same ? ou[1] : ou[0], ou[1], same ? ou[0] : ou[1]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            va[i] = min(qa[i], qb[i]);
            vb[i] = max(qa[i], qb[i]);
        }
        tri[0][0] = 0;
        tri[0][1] = 1;
        tri[0][2] = 2;
        tri[1][0] = 0;
        tri[1][1] = 2;
        tri[1][2] = 3;
    }
    for (int t = 0; t < n_tri; ++t) {
        const unsigned long long idx = out->next++;
        if (idx >= out->limit) continue;         // counted, not written: the caller's buffer is full
        float* pos = out->pos + 9 * idx;
        int* key = out->key ? out->key + 12 * idx : nullptr;   // vertex names are optional
#pragma unroll
        for (int v = 0; v < 3; ++v) {
            const int e = tri[t][v];
            put_vertex(L, c[va[e]], c[vb[e]], gx, gy, gz, vs, pos + 3 * v, key ? key + 4 * v : nullptr);
        }
    }
    return n_tri;
}

// Pool index of a block key (kNoIndex if absent): linear probing from the
// home slot to the key or an empty slot, read-only (extraction leaves the
// volume's counters alone, whatever probe limit it was configured with).
__device__ __forceinline__ unsigned int find_block(const VolumeArgs& vol, unsigned long long key) {
    unsigned int slot = home_slot(key, vol.mask);
    for (unsigned int probes = 0; probes <= vol.mask; ++probes) {
        const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(vol.table + slot);
        if (e.x == key) return (unsigned int)e.y < vol.capacity ? (unsigned int)e.y : kNoIndex;
        if (e.x == kEmptyKey) return kNoIndex;
        slot = (slot + 1) & vol.mask;
    }
    return kNoIndex;
}

// Extract one block (table slot `slot`): stage its lattice, count, reserve,
// write.  Called by the whole workgroup.
__device__ void extract_block(MeshLds& L, const VolumeArgs& vol, unsigned int slot, unsigned long long* counter,
                              float* pos, int* key, unsigned long long max_triangles) {
    const int tid = threadIdx.x;
    const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(vol.table + slot);
    int bx, by, bz;
    unpack_key(e.x, bx, by, bz);
    // the block and its neighbours at +x, +y, +z (and their sums), through the table
    if (tid < 8) {
        unsigned int idx = (unsigned int)e.y;
        if (tid) {
            const int nx = bx + (tid & 1), ny = by + ((tid >> 1) & 1), nz = bz + ((tid >> 2) & 1);
            idx = kNoIndex;
            if (nx < (1 << 20) && ny < (1 << 20) && nz < (1 << 20))   // a key holds blocks below 2^20
                idx = find_block(vol, block_key(nx * 8, ny * 8, nz * 8));
        }
        L.nb[tid] = idx;
    }
    __syncthreads();
    for (int l = tid; l < kLattice; l += kMeshThreads) {
        const int x = l % kSide, y = (l / kSide) % kSide, z = l / (kSide * kSide);
        const int n = (x >> 3) | ((y >> 3) << 1) | ((z >> 3) << 2);
        const unsigned int b = L.nb[n];
        float mean = 0.0f;
        unsigned char fl = 0;
        if (b < vol.capacity) {
            const size_t off = (size_t)b * kBlockVoxels + ((x & 7) | ((y & 7) << 3) | ((z & 7) << 6));
            const float w = vol.weight[off];
            if (w > 0.0f) {
                const float sum = vol.tsdf[off];
                mean = sum / w;
                fl = kObserved | (sum < 0.0f ? kInside : 0);
            }
        }
        L.v[l] = mean;
        L.flag[l] = fl;
    }
    __syncthreads();
    // two cells per thread: count, reserve, write
    int count = 0;
    for (int c = tid; c < kBlockVoxels; c += kMeshThreads) {
        const int x = c & 7, y = (c >> 3) & 7, z = c >> 6;
        for (int t = 0; t < 6; ++t) count += tet_triangles(L, x, y, z, 0, 0, 0, t, vol.vs, nullptr);
    }
    const unsigned int incl = wave_inclusive_sum((unsigned int)count);
    const int wave = tid >> 6, lane = tid & 63;
    if (lane == 63) L.scan[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        unsigned long long acc = 0;
        for (int w = 0; w < kMeshThreads / 64; ++w) {
            const unsigned int t = L.scan[w];
            L.scan[w] = (unsigned int)acc;
            acc += t;
        }
        L.base = acc ? atomicAdd(counter, acc) : 0ull;
    }
    __syncthreads();
    if (count) {
        TriOut out;
        out.pos = pos;
        out.key = key;
        out.next = L.base + L.scan[wave] + incl - (unsigned int)count;
        out.limit = max_triangles;
        const int gx0 = bx * 8, gy0 = by * 8, gz0 = bz * 8;
        for (int c = tid; c < kBlockVoxels; c += kMeshThreads) {
            const int x = c & 7, y = (c >> 3) & 7, z = c >> 6;
            for (int t = 0; t < 6; ++t) tet_triangles(L, x, y, z, gx0 + x, gy0 + y, gz0 + z, t, vol.vs, &out);
        }
    }
    __syncthreads();                               // L is restaged for the next block
}

// Workgroups take 256-slot stretches of the table in turn; a stretch's
// blocks (slots holding a pool index) are listed in LDS and extracted one
// after another.
__global__ __launch_bounds__(kMeshThreads) void k_mesh(VolumeArgs vol, unsigned long long n_entries,
                                                       unsigned long long* counter, float* pos, int* key,
                                                       unsigned long long max_triangles) {
    __shared__ MeshLds L;
    __shared__ unsigned int s_list[kMeshThreads];
    __shared__ unsigned int s_n;
    for (unsigned long long c0 = (unsigned long long)blockIdx.x * kMeshThreads; c0 < n_entries;
         c0 += (unsigned long long)gridDim.x * kMeshThreads) {
        if (threadIdx.x == 0) s_n = 0;
        __syncthreads();
        const unsigned long long i = c0 + threadIdx.x;
        if (i < n_entries) {
            const ulonglong2 e = *reinterpret_cast<const ulonglong2*>(vol.table + i);
            if (e.x != kEmptyKey && (unsigned int)e.y < vol.capacity) s_list[atomicAdd(&s_n, 1u)] = (unsigned int)i;
        }
        __syncthreads();
        const unsigned int n = s_n;
        for (unsigned int j = 0; j < n; ++j) extract_block(L, vol, s_list[j], counter, pos, key, max_triangles);
        __syncthreads();                           // every thread has read s_n before it is cleared
    }
}

__global__ void k_mesh_clear(unsigned long long* counter) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *counter = 0;
}

}  // namespace

bool launch_mesh(const VolumeArgs& v, unsigned long long table_entries, unsigned long long* counter, float* pos,
                 int* key, unsigned long long max_triangles, hipStream_t s) {
    unsigned long long g = (table_entries + kMeshThreads - 1) / kMeshThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    hipLaunchKernelGGL(k_mesh_clear, dim3(1), dim3(64), 0, s, counter);
    hipLaunchKernelGGL(k_mesh, dim3((unsigned int)g), dim3(kMeshThreads), 0, s, v, table_entries, counter, pos, key,
                       max_triangles);
    return hipGetLastError() == hipSuccess;
}

}  // namespace tsdf
