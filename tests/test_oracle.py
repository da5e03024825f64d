"""The oracle against what the pages and geometry fix (CPU only).

Every check lives in tests/oracle_pins.py so that the mutation tests can run
the same checks against copies of the oracle with a planted mistake.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_oracle():
    oracle.build()


@pytest.mark.parametrize("pin", sorted(oracle_pins.PINS))
def test_pin(pin):
    failures = oracle_pins.PINS[pin]()
    assert failures == [], failures


@pytest.mark.parametrize("pin", sorted(oracle_pins.MESH_PINS))
def test_mesh_pin(pin):
    failures = oracle_pins.MESH_PINS[pin]()
    assert failures == [], failures


def test_plane_every_voxel_single_ray():
    # 2 cm pixel footprint on 1 cm voxels: every kept voxel receives one ray,
    # so its colour is exactly one pixel's colour / 255
    from hash_table_amd import scenes
    wl = scenes.workload("plane64x48")
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity)
    o.integrate(wl.frame(0))
    s = o.block_sums(o.block_coords())
    w = s["weight"]
    assert set(np.unique(w[w > 0])) == {1.0}
    vals = np.round(s["r"][w > 0] * 255.0, 9)
    assert np.all(vals == np.round(vals))


# ---------------------------------------------------------------------------
# mutation tests: each plants one plausible mistake in a copy of the oracle
# source; some pin must fail (or the mutant must crash).
# ---------------------------------------------------------------------------
MUTATIONS = [
    # (name, original text, replacement, occurrences, pins expected to notice)
    ("distance at cell corner, not centre", "((float)k[i] + 0.5f) * vs", "((float)k[i] + 0.0f) * vs", 1,
     "plane,sphere"),
    ("sdf sign flipped", "const float sdf = d - zc;", "const float sdf = zc - d;", 1, "plane"),
    ("occlusion test dropped", "if (sdf >= -trunc && sdf <= trunc)", "if (sdf <= trunc)", 1,
     "plane,bruteforce"),
    ("band test dropped", "if (sdf >= -trunc && sdf <= trunc)", "if (sdf >= -trunc)", 1, "plane,bruteforce"),
    ("walk skips cells", "k[m] += step[m];", "k[m] += 2 * step[m];", 1, "bruteforce,plane"),
    ("wrong first boundary", "tmax[i] = ((float)(k[i] + 1) - gA[i]) * inv[i];",
     "tmax[i] = ((float)k[i] - gA[i]) * inv[i];", 1, "bruteforce"),
    ("walk stops half way", "if (!(tmax[m] <= 1.0f)) break;", "if (!(tmax[m] <= 0.5f)) break;", 1,
     "bruteforce,plane"),
    ("rotation transposed", "((R[3 * i + 0] * a[0] + R[3 * i + 1] * a[1]) + R[3 * i + 2] * a[2])",
     "((R[i] * a[0] + R[3 + i] * a[1]) + R[6 + i] * a[2])", 1, "bruteforce"),
    ("fx used for rows", "((float)v - cy) / fy", "((float)v - cy) / fx", 1, "bruteforce"),
    ("tsdf not normalised", "(double)sdf / (double)o->trunc", "(double)sdf", 1, "plane,bruteforce"),
    ("colour scale", "(double)col[0] / 255.0", "(double)col[0] / 256.0", 1, "bruteforce"),
    ("block index truncates toward zero", "if (k % kBlockEdge != 0 && k < 0) q -= 1;", "", 1, "plane"),
    ("capacity off by one", "(int64_t)o->blocks.size() >= o->capacity", "(int64_t)o->blocks.size() > o->capacity",
     1, "invariants"),
    ("near points used", "if (d <= trunc) { s.near_skipped++; continue; }", "", 1, "edges"),
    ("range check dropped", "in_range = false;", "in_range = true;", 1, "edges"),
    ("voxel index axes swapped", "(k[0] - kBlockEdge * bc.x) + kBlockEdge * (k[1] - kBlockEdge * bc.y) +\n"
     "                      kBlockEdge * kBlockEdge * (k[2] - kBlockEdge * bc.z)",
     "(k[2] - kBlockEdge * bc.z) + kBlockEdge * (k[1] - kBlockEdge * bc.y) +\n"
     "                      kBlockEdge * kBlockEdge * (k[0] - kBlockEdge * bc.x)", 1, "plane"),
    ("weight of two", "S.weight[local] += 1.0;", "S.weight[local] += 2.0;", 1, "plane,bruteforce"),
    # the reprojection reading of the occlusion test (C8)
    ("projection rounds down", "((xc / zc) * fx + cx) + 0.5f", "((xc / zc) * fx + cx) + 0.0f", 1, "reprojection"),
    ("hidden when in front", "return zc - D > trunc;", "return D - zc > trunc;", 1, "reprojection"),
    ("projection uses rotation rows", "const float xc = (R[0] * q0 + R[3] * q1) + R[6] * q2;",
     "const float xc = (R[0] * q0 + R[1] * q1) + R[2] * q2;", 1, "reprojection"),
    # the measurement counts (per frame and per call)
    ("U counts a voxel's first touch only", "if (blk.voxel_frame && blk.voxel_frame[local] != stamp) {",
     "if (blk.voxel_frame && blk.voxel_frame[local] == 0) {", 1, "counters"),
    ("cells counted twice", "s.cells_visited++;", "s.cells_visited += 2;", 1, "counters"),
    ("B_t counts new blocks only", "if (blk.block_frame != stamp) {", "if (blk.block_frame == 0) {", 1,
     "counters"),
    ("call's B counts new blocks only", "if (blk.block_call != o->call) {", "if (blk.block_call == 0) {", 1,
     "counters"),
    ("call's fresh and old voxels swapped", "if (blk.created_call == o->call)",
     "if (blk.created_call != o->call)", 1, "counters"),
]


# the extraction oracle (mesh_oracle.cpp)
MESH_MUTATIONS = [
    ("interpolation from the wrong end", "const double t = p.v / (p.v - q.v);",
     "const double t = q.v / (q.v - p.v);", 1, "mesh_fields,mesh_plane"),
    ("inside where the sum is positive", "c.inside = tsdf[q] < 0.0;", "c.inside = tsdf[q] > 0.0;", 1,
     "mesh_fields,mesh_plane"),
    ("one tetrahedron's orientation wrong", "kOrderSign[6] = {+1, -1, -1, +1, +1, -1};",
     "kOrderSign[6] = {+1, -1, -1, -1, +1, -1};", 1, "mesh_fields"),
    ("a tetrahedron missing, another twice", "{2, 0, 1}, {2, 1, 0}};", "{2, 0, 1}, {2, 0, 1}};", 1,
     "mesh_fields,mesh_plane"),
    ("unobserved voxels used", "if (!(weight[q] > 0.0)) return false;", "if (!(weight[q] >= 0.0)) return false;",
     1, "mesh_fields"),
    ("lone outside corner faces inwards", "const bool fwd = (perm_sign(perm) * s > 0) == (ni == 1);",
     "const bool fwd = perm_sign(perm) * s > 0;", 1, "mesh_fields"),
    ("block of a negative voxel truncated", "k[0] >= 0 ? k[0] / kEdge : -((-k[0] + kEdge - 1) / kEdge)",
     "k[0] / kEdge", 1, "mesh_fields"),
    ("vertex at the edge midpoint", "m->vpos.push_back(P + t * (Q - P));", "m->vpos.push_back(P + 0.5 * (Q - P));",
     1, "mesh_fields,mesh_plane,mesh_sphere"),
]


def _run_mutant(tmp_path, source, old, new, count, pins, output="libmutant.so"):
    src = open(source).read()
    assert src.count(old) == count, f"mutation target not found: {old!r}"
    mutant = tmp_path / "mutant.cpp"
    mutant.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant), str(tmp_path / output))
    return subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib, pins],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


@pytest.mark.parametrize("name,old,new,count,pins", MESH_MUTATIONS, ids=[m[0] for m in MESH_MUTATIONS])
def test_mesh_mutant_is_caught(tmp_path, name, old, new, count, pins):
    proc = _run_mutant(tmp_path, oracle.MESH_SOURCE, old, new, count, pins, "libmeshmutant.so")
    if proc.returncode != 0:
        return                                     # the mutant crashed: caught
    result = json.loads(proc.stdout.strip().splitlines()[-1])
    caught = {p: f for p, f in result.items() if f}
    assert caught, f"mutation '{name}' passed every pin: {result}"


@pytest.mark.parametrize("name,old,new,count,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new, count, pins):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == count, f"mutation target not found: {old!r}"
    mutant = tmp_path / "mutant.cpp"
    mutant.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant), str(tmp_path / "libmutant.so"))
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib, pins],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)
    if proc.returncode != 0:
        return                                     # the mutant crashed: caught
    result = json.loads(proc.stdout.strip().splitlines()[-1])
    caught = {p: f for p, f in result.items() if f}
    assert caught, f"mutation '{name}' passed every pin: {result}"
