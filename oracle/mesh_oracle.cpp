/*
 * mesh_oracle.cpp -- reference ("oracle") surface extraction for
 * hash-blocked TSDF volumes.  TEST INFRASTRUCTURE ONLY: the tests and the
 * smoke check use it to check the HIP library's extraction kernel; the HIP
 * library never links, loads or calls it, and the two share no code.
 *
 * "What Irregularity Costs: CUDA C++, Rust, and Triton on a Hash-Blocked GPU
 * Workload", section 3, extracts the surface once, after integration, by
 * marching tetrahedra over the fused volume; its section 3a gates results on
 * the extracted surface (a sphere within a quarter voxel; distances between
 * vertex sets).  The pages name the method only; this file writes it out
 * with these conventions (the HIP kernel follows the same written rules,
 * independently):
 *
 *   M1  samples sit at voxel centres, world position (k + 1/2) vs per axis;
 *       a voxel is observed iff its weight sum is > 0, its value is the mean
 *       TSDF (sum / weight).
 *   M2  the cell with lower corner at voxel k spans voxels k + {0,1}^3; it is
 *       cut into six tetrahedra along its main diagonal: for each ordering
 *       (a, b, c) of the axes, in the order xyz, xzy, yxz, yzx, zxy, zyx, the
 *       tetrahedron with corners P0 = k, P1 = k + e_a, P2 = k + e_a + e_b,
 *       P3 = k + (1, 1, 1).  Neighbouring cells cut their shared face along
 *       the same diagonal, so the tetrahedra tile space.  A tetrahedron is
 *       used iff its four corners are observed.
 *   M3  a corner is inside iff its TSDF sum is < 0 (behind the surface).
 *   M4  each edge of a used tetrahedron with one corner inside and one
 *       outside holds one vertex.  Every such edge runs from a lattice point
 *       p to p + d, d in {0,1}^3 without 0 (corners with a lower index are
 *       never higher on any axis); the vertex is named (p, d) and lies at
 *       P + t (Q - P), t = v_p / (v_p - v_q), P and Q the two corners' world
 *       positions, v their means.
 *   M5  triangles, oriented so that (B - A) x (C - A) points from inside to
 *       outside: with the tetrahedron's orientation s = the sign of the
 *       ordering (a, b, c) (+1 for xyz, yzx, zxy),
 *         one inside corner i, others j < k < l: (ij, ik, il) if
 *           sign(i, j, k, l) s > 0, else (ij, il, ik);
 *         one outside corner o, others j < k < l: the reverse, (oj, ol, ok)
 *           if sign(o, j, k, l) s > 0, else (oj, ok, ol);
 *         two inside i0 < i1, two outside o0 < o1: the quad
 *           (i0o0, i0o1, i1o1, i1o0) if sign(i0, i1, o0, o1) s > 0, else
 *           (i0o0, i1o0, i1o1, i0o1), cut into (V0, V1, V2) and (V0, V2, V3);
 *       sign(...) is the sign of the permutation of the corner indices
 *       0..3, and xy the vertex on the edge between corners x and y.
 *
 * Blocks are visited in ascending coordinate order, cells in voxel-index
 * order, tetrahedra in the order of M2.  Arithmetic in double.
 */
#include <cstdint>
#include <cstring>
#include <map>
#include <tuple>
#include <vector>

namespace {

constexpr int kEdge = 8;
constexpr int kVoxels = kEdge * kEdge * kEdge;

struct Coord {
    int32_t x, y, z;
    bool operator<(const Coord& o) const { return std::tie(x, y, z) < std::tie(o.x, o.y, o.z); }
};

struct VertexKey {
    int32_t x, y, z, d;
    bool operator<(const VertexKey& o) const { return std::tie(x, y, z, d) < std::tie(o.x, o.y, o.z, o.d); }
};

struct Mesh {
    std::map<VertexKey, int64_t> vindex;       // key -> index in creation order
    std::vector<VertexKey> vkey;
    std::vector<double> vpos;                  // 3 per vertex
    std::vector<int64_t> tri;                  // 3 per triangle (creation-order vertex indices)
};

// sign of the permutation (p0, p1, p2, p3) of 0..3
int perm_sign(const int p[4]) {
    int s = 1;
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (p[i] > p[j]) s = -s;
    return s;
}

const int kOrder[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
const int kOrderSign[6] = {+1, -1, -1, +1, +1, -1};

struct Corner {
    int32_t k[3];      // voxel coordinate
    double v;          // mean TSDF
    bool inside;
};

}  // namespace

extern "C" {

/* Extract the surface of a volume given as n blocks: coords (n x 3 block
 * coordinates), tsdf and weight sums (n x 512 each, voxel x + 8 y + 64 z).
 * vs: voxel size in metres.  Returns a handle (oracle_mesh_destroy). */
void* oracle_mesh(const int32_t* coords, const double* tsdf, const double* weight, int64_t n, double vs) {
    std::map<Coord, int64_t> blocks;
    for (int64_t i = 0; i < n; ++i) blocks[Coord{coords[3 * i], coords[3 * i + 1], coords[3 * i + 2]}] = i;
    Mesh* m = new Mesh();

    // M1: the sample at voxel k, if observed
    auto sample = [&](const int32_t k[3], Corner& c) -> bool {
        const int32_t b[3] = {k[0] >= 0 ? k[0] / kEdge : -((-k[0] + kEdge - 1) / kEdge),
                              k[1] >= 0 ? k[1] / kEdge : -((-k[1] + kEdge - 1) / kEdge),
                              k[2] >= 0 ? k[2] / kEdge : -((-k[2] + kEdge - 1) / kEdge)};
        auto it = blocks.find(Coord{b[0], b[1], b[2]});
        if (it == blocks.end()) return false;
        const int local = (k[0] - kEdge * b[0]) + kEdge * (k[1] - kEdge * b[1]) + kEdge * kEdge * (k[2] - kEdge * b[2]);
        const int64_t q = it->second * kVoxels + local;
        if (!(weight[q] > 0.0)) return false;
        std::memcpy(c.k, k, sizeof(c.k));
        c.v = tsdf[q] / weight[q];
        c.inside = tsdf[q] < 0.0;                                        // M3
        return true;
    };
    // M4: the vertex on the edge between corners p (lower) and q
    auto vertex = [&](const Corner& p, const Corner& q) -> int64_t {
        const int32_t d = (q.k[0] - p.k[0]) | ((q.k[1] - p.k[1]) << 1) | ((q.k[2] - p.k[2]) << 2);
        const VertexKey key{p.k[0], p.k[1], p.k[2], d};
        auto it = m->vindex.find(key);
        if (it != m->vindex.end()) return it->second;
        const double t = p.v / (p.v - q.v);
        const int64_t id = (int64_t)m->vkey.size();
        m->vkey.push_back(key);
        for (int a = 0; a < 3; ++a) {
            const double P = ((double)p.k[a] + 0.5) * vs, Q = ((double)q.k[a] + 0.5) * vs;
            m->vpos.push_back(P + t * (Q - P));
        }
        m->vindex.emplace(key, id);
        return id;
    };
    auto tri = [&](int64_t a, int64_t b, int64_t c) {
        m->tri.push_back(a);
        m->tri.push_back(b);
        m->tri.push_back(c);
    };

    for (const auto& kv : blocks) {                   // ascending coordinates
        const Coord bc = kv.first;
        for (int local = 0; local < kVoxels; ++local) {
            const int32_t base[3] = {bc.x * kEdge + (local & 7), bc.y * kEdge + ((local >> 3) & 7),
                                     bc.z * kEdge + (local >> 6)};
            for (int o = 0; o < 6; ++o) {              // M2
                Corner P[4];
                int32_t k[3] = {base[0], base[1], base[2]};
                bool ok = sample(k, P[0]);
                for (int s = 0; s < 3 && ok; ++s) {
                    k[kOrder[o][s]] += 1;
                    ok = sample(k, P[s + 1]);
                }
                if (!ok) continue;
                int in[4], out[4], ni = 0, no = 0;
                for (int c = 0; c < 4; ++c) {
                    if (P[c].inside) in[ni++] = c; else out[no++] = c;
                }
                if (ni == 0 || ni == 4) continue;
                const int s = kOrderSign[o];
                auto V = [&](int x, int y) { return x < y ? vertex(P[x], P[y]) : vertex(P[y], P[x]); };
                if (ni == 1 || ni == 3) {                  // M5: one corner against three
                    const int lone = ni == 1 ? in[0] : out[0];
                    int rest[3], r = 0;
                    for (int c = 0; c < 4; ++c)
                        if (c != lone) rest[r++] = c;
                    const int perm[4] = {lone, rest[0], rest[1], rest[2]};
                    const bool fwd = (perm_sign(perm) * s > 0) == (ni == 1);
                    if (fwd)
                        tri(V(lone, rest[0]), V(lone, rest[1]), V(lone, rest[2]));
                    else
                        tri(V(lone, rest[0]), V(lone, rest[2]), V(lone, rest[1]));
                } else {                                   // M5: two against two
                    const int i0 = in[0], i1 = in[1], o0 = out[0], o1 = out[1];
                    const int perm[4] = {i0, i1, o0, o1};
                    int64_t q[4];
                    if (perm_sign(perm) * s > 0) {
                        q[0] = V(i0, o0); q[1] = V(i0, o1); q[2] = V(i1, o1); q[3] = V(i1, o0);
                    } else {
                        q[0] = V(i0, o0); q[1] = V(i1, o0); q[2] = V(i1, o1); q[3] = V(i0, o1);
                    }
                    tri(q[0], q[1], q[2]);
                    tri(q[0], q[2], q[3]);
                }
            }
        }
    }
    return m;
}

int64_t oracle_mesh_vertex_count(void* h) { return (int64_t)static_cast<Mesh*>(h)->vkey.size(); }
int64_t oracle_mesh_triangle_count(void* h) { return (int64_t)static_cast<Mesh*>(h)->tri.size() / 3; }

/* Vertices in creation order: keys (nv x 4: lattice point x, y, z and the
 * direction d = dx | dy << 1 | dz << 2) and positions (nv x 3, metres). */
void oracle_mesh_vertices(void* h, int32_t* keys, double* pos) {
    const Mesh* m = static_cast<Mesh*>(h);
    for (size_t i = 0; i < m->vkey.size(); ++i) {
        keys[4 * i + 0] = m->vkey[i].x;
        keys[4 * i + 1] = m->vkey[i].y;
        keys[4 * i + 2] = m->vkey[i].z;
        keys[4 * i + 3] = m->vkey[i].d;
    }
    std::memcpy(pos, m->vpos.data(), sizeof(double) * m->vpos.size());
}

/* Triangles (nt x 3 vertex indices into the creation-order vertex list). */
void oracle_mesh_triangles(void* h, int64_t* tris) {
    const Mesh* m = static_cast<Mesh*>(h);
    std::memcpy(tris, m->tri.data(), sizeof(int64_t) * m->tri.size());
}

void oracle_mesh_destroy(void* h) { delete static_cast<Mesh*>(h); }

}  // extern "C"
