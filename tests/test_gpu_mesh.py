"""Surface extraction (marching tetrahedra) on the GPU against the extraction
oracle (needs an MI355X).

Two comparisons: on the same fused volume (the GPU's, exported), every
triangle -- its three vertex names in order -- must be identical and every
position within float32 rounding; and along the independent chain (the
oracle integrates and extracts; the GPU integrates and extracts), vertex
names must agree wherever neither end of the edge is within the 1e-4 mean
tolerance of zero, with positions within what that tolerance allows; the
mean and Hausdorff distances between the vertex sets are reported (the
paper's cross-arm metric).  The analytic gates run on the GPU's own surface:
the plane at z = 1.000 m and the sphere within a quarter voxel.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from hash_table_amd import scenes
from tests import oracle_pins, parity
from tests.parity import say

pytestmark = pytest.mark.gpu
TIE = parity.MEAN_TOL           # |mean| below this: the two sides may disagree on the side


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build()


def _rows(keys):
    """(n, 3, 4) vertex names -> one void row of 48 bytes per triangle."""
    k = np.ascontiguousarray(keys, np.int32).reshape(len(keys), 12)
    return k.view(np.dtype((np.void, 48))).ravel()


def _oracle_triangles(m):
    return m.keys[m.tris], m.pos[m.tris]           # (nt, 3, 4), (nt, 3, 3)


def _pos_tol(p):
    """float32 rounding of a vertex position: a few spacings of the largest
    coordinate (P, Q and t (Q - P) each rounded)."""
    return 8.0 * np.spacing(np.float32(np.abs(p).max())) + 1e-9


def compare_same_volume(gk, gp, ok, op, label):
    """Triangle multisets equal (vertex names in order); positions close."""
    assert len(gk) == len(ok), f"{label}: {len(gk)} triangles on the GPU, {len(ok)} in the oracle"
    gr, orr = _rows(gk), _rows(ok)
    gi, oi = np.argsort(gr, kind="stable"), np.argsort(orr, kind="stable")
    assert np.array_equal(gr[gi], orr[oi]), f"{label}: the triangle sets differ"
    d = np.abs(gp[gi].astype(np.float64) - op[oi]).max() if len(gi) else 0.0
    tol = _pos_tol(op)
    say(f"  {label}: {len(gk)} triangles identical, largest position difference {d:.3g} m (tolerance {tol:.3g})")
    assert d <= tol


def _vertex_table(keys, pos):
    """Unique vertices: {name tuple: position} from triangle soups."""
    k = np.ascontiguousarray(keys, np.int32).reshape(-1, 4)
    p = np.asarray(pos, np.float64).reshape(-1, 3)
    u, first = np.unique(k, axis=0, return_index=True)
    return u, p[first]


def _pack_lattice(k):
    """Lattice points (n, 3), |coordinate| < 2^19, as sortable int64."""
    k = np.asarray(k, np.int64).reshape(-1, 3)
    assert np.abs(k).max(initial=0) < (1 << 19)
    k = k + (1 << 19)
    return k[:, 0] | (k[:, 1] << 20) | (k[:, 2] << 40)


def _pack_vertex(keys):
    """Vertex names (n, 4): lattice point and direction, as int64."""
    return _pack_lattice(keys[:, :3]) | (np.asarray(keys[:, 3], np.int64) << 60)


def _gpu_volume(frames, vs, tr, cap, batch=16):
    vol, st, coords, arrays, _ = parity.gpu_integrate(frames, vs, tr, cap, batch=batch,
                                                      max_batch_pixels=batch * frames[0].width * frames[0].height)
    return vol, st, coords, arrays


def _cases():
    wl = scenes.workload("spherewall320x240_noisefree")
    room = scenes.workload("room640x480")
    return {
        "dense_plane": ([oracle_pins._dense_plane()], 0.01, 0.04, 1 << 16),
        "sphere": (list(wl.frames()), wl.voxel_size, wl.trunc, wl.pool_capacity),
        "room16": (list(room.frames(0, 16)), room.voxel_size, room.trunc, room.pool_capacity),
    }


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["dense_plane", "sphere", "room16"])
def test_mesh_parity(name):
    frames, vs, tr, cap = _cases()[name]
    say(f"  {name}: gpu integrate + extract")
    vol, st, coords, arrays = _gpu_volume(frames, vs, tr, cap)
    gp, gk = vol.extract_mesh()
    # 1. the same fused volume: the GPU's sums through the extraction oracle
    m = oracle.extract_mesh(coords, arrays["tsdf"].astype(np.float64), arrays["weight"].astype(np.float64), vs)
    ok, op = _oracle_triangles(m)
    compare_same_volume(gk, gp, ok, op, f"{name} (same volume)")
    # 2. the independent chain: the oracle's own integration and extraction
    o = parity.oracle_integrate(frames, vs, tr, cap)
    oc = o.block_coords()
    s = o.block_sums(oc)
    mo = oracle.extract_mesh(oc, s["tsdf"], s["weight"], vs)
    gu, gpos = _vertex_table(gk, gp)
    ou, opos = mo.keys, mo.pos
    # the oracle's mean at both ends of every vertex's edge, to find ties
    kk, flat = oracle_pins._voxel_table(o, oc)
    vkeys = _pack_lattice(kk)
    order = np.argsort(vkeys)
    vkeys, vmean = vkeys[order], (flat["tsdf"] / flat["weight"])[order]

    def end_means(keys):
        p = keys[:, :3].astype(np.int64)
        d = keys[:, 3].astype(np.int64)
        q = p + np.stack([d & 1, (d >> 1) & 1, (d >> 2) & 1], 1)
        out = []
        for e in (p, q):
            pk = _pack_lattice(e)
            i = np.clip(np.searchsorted(vkeys, pk), 0, len(vkeys) - 1)
            out.append(np.where(vkeys[i] == pk, vmean[i], 0.0))      # unobserved: no vertex either side
        return out

    gkey, okey = _pack_vertex(gu), _pack_vertex(ou)
    in_o = np.isin(gkey, okey)
    in_g = np.isin(okey, gkey)
    mg = end_means(gu)
    mo_ = end_means(ou)
    tie_g = (np.abs(mg[0]) <= TIE) | (np.abs(mg[1]) <= TIE)
    tie_o = (np.abs(mo_[0]) <= TIE) | (np.abs(mo_[1]) <= TIE)
    only_g, only_o = int((~in_o & ~tie_g).sum()), int((~in_g & ~tie_o).sum())
    assert only_g == 0 and only_o == 0, f"{name}: vertex sets differ on clear edges ({only_g}, {only_o})"
    # positions: t = v_p / (v_p - v_q) moves by at most (e_p + e_q) / |v_p - v_q|
    # for mean errors e <= 1e-4, times the edge length, plus float rounding
    gi = np.nonzero(in_o)[0]
    oi = np.searchsorted(okey, gkey[gi], sorter=np.argsort(okey))
    oi = np.argsort(okey)[oi]
    d = np.linalg.norm(gpos[gi] - opos[oi], axis=1)
    gap = np.abs(mg[0][gi] - mg[1][gi])
    length = vs * np.sqrt([bin(int(x)).count("1") for x in gu[gi, 3]])
    bound = 2 * TIE / np.maximum(gap, 2 * TIE) * length + _pos_tol(opos)
    assert np.all(d <= bound), f"{name}: a vertex {d.max():.3g} m from the oracle's"
    # the pages' cross-arm metric: mean and Hausdorff distance between the vertex sets
    from scipy.spatial import cKDTree
    d_go = cKDTree(opos).query(gpos)[0]
    d_og = cKDTree(gpos).query(opos)[0]
    say(f"  {name} (independent chain): {len(gu)} GPU vertices, {len(ou)} oracle vertices, "
        f"{len(gi)} shared, {int(tie_g.sum())} on tie edges; largest shared-vertex difference {d.max():.3g} m; "
        f"mean distance {np.concatenate([d_go, d_og]).mean():.3g} m, Hausdorff {max(d_go.max(), d_og.max()):.3g} m")
    assert st["update_misses"] == 0


def test_mesh_gates_on_gpu_surface():
    """The analytic gates on the GPU's own surface: the dense plane's vertices
    at z = 1.000 m, the noise-free sphere's front cap within a quarter voxel
    of r = 0.5 m at (0, 0, 1.5)."""
    frames, vs, tr, cap = _cases()["dense_plane"]
    vol, *_ = _gpu_volume(frames, vs, tr, cap)
    gp, gk = vol.extract_mesh()
    z = gp[..., 2].astype(np.float64)
    say(f"  plane: {len(gp)} triangles, z within {np.abs(z - 1.0).max():.3g} m of 1.000")
    assert len(gp) > 1000 and np.abs(z - 1.0).max() < 1e-6
    assert np.all(gk[..., 2] == 99) and np.all(gk[..., 3] & 4)
    frames, vs, tr, cap = _cases()["sphere"]
    vol, *_ = _gpu_volume(frames, vs, tr, cap)
    gp, _ = vol.extract_mesh()
    p = gp.reshape(-1, 3).astype(np.float64)
    cap_v = (p[:, 2] < 1.2) & (np.hypot(p[:, 0], p[:, 1]) < 0.2)
    d = np.abs(np.linalg.norm(p[cap_v] - np.array([0.0, 0.0, 1.5]), axis=1) - 0.5)
    say(f"  sphere cap: {int(cap_v.sum())} vertex uses, largest distance {d.max() * 1000:.3f} mm, "
        f"mean {d.mean() * 1000:.3f} mm (gate {vs / 4 * 1000:.2f} mm)")
    assert cap_v.sum() > 500 and d.max() <= vs / 4


def test_mesh_output_limits():
    """Too small an output buffer: the count is exact, TSDF_ESMALL, only the
    first max_triangles written; a count-only call; an empty volume."""
    import torch
    from hash_table_amd import tsdf
    frames, vs, tr, cap = _cases()["sphere"]
    vol, *_ = _gpu_volume(frames[:2], vs, tr, cap)
    gp, _ = vol.extract_mesh()
    n = len(gp)
    assert n > 100
    sh = torch.cuda.current_stream().cuda_stream
    with pytest.raises(tsdf.TsdfError) as e:                            # count only
        tsdf.tsdf_extract_mesh(vol.handle, 0, 0, 0, sh)
    assert e.value.status == tsdf.TSDF_ESMALL and e.value.n_triangles == n
    pos = torch.full((17, 9), -7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_extract_mesh(vol.handle, pos.data_ptr(), 0, 16, sh)
    assert e.value.status == tsdf.TSDF_ESMALL and e.value.n_triangles == n
    got = pos.cpu().numpy()
    assert np.all(got[16] == -7.0) and np.all(got[:16] != -7.0)          # 16 written, the 17th untouched
    empty = tsdf.Volume(vs, tr, 64)
    assert tsdf.tsdf_extract_mesh(empty.handle, 0, 0, 0, sh) == 0
    with pytest.raises(tsdf.TsdfError):
        tsdf.tsdf_extract_mesh(vol.handle, 0, 0, 5, sh)                   # no buffer for 5 triangles


@pytest.mark.timeout(600)
def test_mesh_room_full_volume():
    """The benchmark's volume (all 100 frames of the 640 x 480 room in one
    call): every triangle identical to the extraction oracle's on the same
    fused volume."""
    wl = scenes.workload("room640x480")
    frames = list(wl.frames())
    vol, st, coords, arrays = _gpu_volume(frames, wl.voxel_size, wl.trunc, wl.pool_capacity, batch=100)
    gp, gk = vol.extract_mesh()
    m = oracle.extract_mesh(coords, arrays["tsdf"].astype(np.float64), arrays["weight"].astype(np.float64),
                            wl.voxel_size)
    ok, op = _oracle_triangles(m)
    compare_same_volume(gk, gp, ok, op, "room640x480 (100 frames)")
