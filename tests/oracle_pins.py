"""Checks that pin the oracle to facts other than itself.

Each ``*_failures(lib)`` function integrates with the oracle library at
``lib`` and returns a list of failure messages (empty = pinned).  They are
shared by the oracle tests and by the mutation tests, which build copies of
the oracle with a planted mistake and require that some check fails.

Run as a script (used by the mutation tests, in a subprocess, so that a
planted mistake that crashes cannot take the test runner down):
    python tests/oracle_pins.py LIB PIN[,PIN...]
prints one JSON object {pin: [failures]}.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from hash_table_amd import scenes  # noqa: E402

try:
    from tests import bruteforce  # noqa: E402
except ImportError:                # run as a script from tests/
    import bruteforce  # type: ignore  # noqa: E402

PLANE_BLOCKS = {(bx, by, 12) for bx in range(-9, 9) for by in range(-7, 6)}


def _voxel_table(o, coords=None):
    """(global voxel index (n,3) int64, sums dict of flat arrays) for every
    voxel with weight > 0."""
    if coords is None:
        coords = o.block_coords()
    s = o.block_sums(coords)
    w = s["weight"]
    bi, li = np.nonzero(w > 0)
    local = np.stack([li % 8, (li // 8) % 8, li // 64], 1)
    k = coords[bi].astype(np.int64) * 8 + local
    flat = {n: a[bi, li] for n, a in s.items()}
    return k, flat


def plane_failures(lib=oracle.LIBRARY):
    """Fronto-parallel plane at z = 1 m, identity pose, vs = 1 cm, trunc = 4 cm.

    Closed form: kept voxels are exactly the layers kz = 96..103 (centres
    0.965..1.035 m, neighbours fail the band by half a voxel); the mean TSDF of
    a voxel is (1 - zc)/0.04; the blocks are {(bx, by, 12): -9 <= bx <= 8,
    -7 <= by <= 5} (the rays of columns 0 and 63 and row 0 reach the outer
    blocks inside the band, row 47 does not reach by = 6)."""
    f = []
    wl = scenes.workload("plane64x48")
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity, library=lib)
    st = o.integrate(wl.frame(0))
    blocks = {tuple(int(x) for x in b) for b in o.block_coords()}
    if blocks != PLANE_BLOCKS:
        f.append(f"plane block set: {len(blocks)} blocks, missing {sorted(PLANE_BLOCKS - blocks)[:4]}, "
                 f"extra {sorted(blocks - PLANE_BLOCKS)[:4]}")
        return f
    k, s = _voxel_table(o)
    layers = set(np.unique(k[:, 2]).tolist())
    if layers != set(range(96, 104)):
        f.append(f"plane layers {sorted(layers)} != 96..103")
    mean = s["tsdf"] / s["weight"]
    zc = (k[:, 2] + 0.5) * 0.01
    expect = (1.0 - zc) / 0.04
    err = np.abs(mean - expect).max() if mean.size else 1.0
    if not err < 2e-5:
        f.append(f"plane mean TSDF off closed form by {err:.3g}")
    if np.any(s["weight"] != np.round(s["weight"])):
        f.append("non-integer weight")
    if int(s["weight"].sum()) != st["voxel_updates"]:
        f.append("sum of weights != voxel updates")
    # linear zero crossing between layers 99 (+0.125) and 100 (-0.125)
    m99 = mean[k[:, 2] == 99].mean()
    m100 = mean[k[:, 2] == 100].mean()
    zx = 0.995 + 0.01 * m99 / (m99 - m100)
    if not abs(zx - 1.0) < 1e-5:
        f.append(f"plane zero crossing {zx:.7f} != 1.0")
    if st["blocks_touched"] != len(PLANE_BLOCKS) or st["blocks_new"] != len(PLANE_BLOCKS):
        f.append("plane block counters")
    if st["points_valid"] != 64 * 48:
        f.append("plane valid points")
    return f


def _single_pixel(frame, u, v):
    depth = np.zeros_like(frame.depth)
    depth[v, u] = frame.depth[v, u]
    return scenes.Frame(depth, frame.rgb, frame.fx, frame.fy, frame.cx, frame.cy, frame.R, frame.t)


def _bf_cases():
    cases = []
    for seed in range(6):
        vs = (0.01, 0.013, 0.005)[seed % 3]
        tr = vs * (4.0, 2.5, 6.0)[seed % 3]
        cases.append((scenes.random_frame(seed, W=7, H=5, translation_scale=0.5), vs, tr))
    return cases


def bruteforce_failures(lib=oracle.LIBRARY, tol=1e-4):
    """Per point and per frame, the oracle's voxels, weights and sums equal a
    brute-force enumeration of the band voxels in double precision (points
    with a decision too close to call in float32 are skipped and counted)."""
    f = []
    n_points = n_ties = 0
    for frame, vs, tr in _bf_cases():
        H, W = frame.depth.shape
        tie_mask = np.zeros((H, W), bool)
        for v in range(H):
            for u in range(W):
                want, tie = bruteforce.point_voxels(frame, u, v, vs, tr)
                if want is None:
                    continue
                n_points += 1
                if tie:
                    n_ties += 1
                    tie_mask[v, u] = True
                    continue
                o = oracle.Oracle(vs, tr, 1 << 20, library=lib)
                o.integrate(_single_pixel(frame, u, v))
                k, s = _voxel_table(o)
                got = {tuple(int(x) for x in kk): i for i, kk in enumerate(k)}
                if set(got) != set(want):
                    f.append(f"point ({u},{v}) vs={vs}: voxel set differs "
                             f"({len(set(got) - set(want))} extra, {len(set(want) - set(got))} missing)")
                    continue
                for kk, (ts, r, g, b) in want.items():
                    i = got[kk]
                    if s["weight"][i] != 1.0:
                        f.append(f"point ({u},{v}): weight {s['weight'][i]}")
                        break
                    d = max(abs(s["tsdf"][i] - ts), abs(s["r"][i] - r), abs(s["g"][i] - g), abs(s["b"][i] - b))
                    if not d < tol:
                        f.append(f"point ({u},{v}) voxel {kk}: sums off by {d:.3g}")
                        break
                if len(f) > 10:
                    return f
        # whole frame, tie points removed: aggregated weights exact, sums close
        depth = frame.depth.copy()
        depth[tie_mask] = 0.0
        fr = scenes.Frame(depth, frame.rgb, frame.fx, frame.fy, frame.cx, frame.cy, frame.R, frame.t)
        want, _ = bruteforce.frame_voxels(fr, vs, tr)
        o = oracle.Oracle(vs, tr, 1 << 20, library=lib)
        o.integrate(fr)
        k, s = _voxel_table(o)
        got = {tuple(int(x) for x in kk): i for i, kk in enumerate(k)}
        if set(got) != set(want):
            f.append(f"frame vs={vs}: voxel sets differ")
            continue
        for kk, acc in want.items():
            i = got[kk]
            if s["weight"][i] != acc[1]:
                f.append(f"frame voxel {kk}: weight {s['weight'][i]} != {acc[1]}")
                break
            d = max(abs(s[n][i] - acc[j]) for j, n in ((0, "tsdf"), (2, "r"), (3, "g"), (4, "b")))
            if not d < tol * acc[1]:
                f.append(f"frame voxel {kk}: sums off by {d:.3g}")
                break
    if n_points < 150:
        f.append(f"only {n_points} brute-force points")
    if n_ties > 0.05 * n_points:
        f.append(f"{n_ties} of {n_points} points are ties")
    return f


def _step_frame():
    """A two-plane step: columns 0-15 of a 24 x 18 image see a wall at 1.013 m,
    the rest one at 2.417 m; random colours, identity pose.  With 0.2 m
    voxels (wider than a pixel there) far-wall cells near the step project
    onto near-wall pixels, some more than trunc behind them (hidden under the
    reprojection reading)."""
    rng = np.random.default_rng(7)
    W, H = 24, 18
    depth = np.full((H, W), 2.417, np.float32)
    depth[:, :16] = 1.013
    rgb = rng.integers(0, 256, size=(H, W, 3), dtype=np.uint8)
    # a slightly turned and shifted camera, so that no ray runs along the grid
    R = scenes.random_rotation(np.random.default_rng(8))
    R = np.linalg.qr(np.eye(3) + 0.05 * (R - R.T))[0]
    R *= np.sign(np.diag(R))[None, :]
    return scenes.Frame(depth, rgb, 20.0, 20.0, (W - 1) / 2.0, (H - 1) / 2.0,
                        R.astype(np.float32), np.array([0.013, -0.021, 0.007], np.float32))


def reprojection_failures(lib=oracle.LIBRARY, tol=1e-4):
    """The reprojection reading of the occlusion test (C8): on frames with
    depth discontinuities (random frames, a two-plane step), every voxel's
    weight lies between the brute-force count of its certain contributions
    and that count plus its float32 ties, and equals it where there is no
    tie; the sums of tie-free voxels match; the step's far band loses cells
    near the step; the fronto-parallel plane is unchanged; and the variant
    never adds a contribution the projective reading lacks."""
    f = []
    cases = [(_step_frame(), 0.2, 0.7)]
    for seed in range(4):
        vs = (0.01, 0.013)[seed % 2]
        cases.append((scenes.random_frame(100 + seed, W=9, H=7, translation_scale=0.5), vs, 4 * vs))
    n_hidden = n_ties = n_kept = 0
    for frame, vs, tr in cases:
        H, W = frame.depth.shape
        want = {}
        ties = {}
        for v in range(H):
            for u in range(W):
                vox, tie_cells = bruteforce.point_voxels(frame, u, v, vs, tr, reproject=True)
                if vox is None:
                    continue
                for kk, (ts, r, g, b) in vox.items():
                    acc = want.setdefault(kk, [0.0, 0.0, 0.0, 0.0, 0.0])
                    for j, x in enumerate((ts, 1.0, r, g, b)):
                        acc[j] += x
                for kk in tie_cells:
                    ties[kk] = ties.get(kk, 0) + 1
        n_ties += sum(ties.values())
        n_kept += int(sum(a[1] for a in want.values()))
        o = oracle.Oracle(vs, tr, 1 << 20, library=lib, reproject=True)
        o.integrate(frame)
        k, s = _voxel_table(o)
        got = {tuple(int(x) for x in kk): i for i, kk in enumerate(k)}
        for kk in set(got) | set(want):
            w_got = float(s["weight"][got[kk]]) if kk in got else 0.0
            acc = want.get(kk)
            w_want = acc[1] if acc else 0.0
            t = ties.get(kk, 0)
            if not (w_want - t <= w_got <= w_want + t):
                f.append(f"vs={vs} voxel {kk}: weight {w_got}, brute force {w_want} (+-{t} ties)")
                break
            if t == 0 and acc and kk in got:
                d = max(abs(s[n][got[kk]] - acc[j]) for j, n in ((0, "tsdf"), (2, "r"), (3, "g"), (4, "b")))
                if not d < tol * acc[1]:
                    f.append(f"vs={vs} voxel {kk}: sums off by {d:.3g}")
                    break
        # the variant only removes contributions
        base = oracle.Oracle(vs, tr, 1 << 20, library=lib)
        base.integrate(frame)
        kb, sb = _voxel_table(base)
        gb = {tuple(int(x) for x in kk): i for i, kk in enumerate(kb)}
        extra = [kk for kk in got if kk not in gb or s["weight"][got[kk]] > sb["weight"][gb[kk]]]
        if extra:
            f.append(f"vs={vs}: the reprojection variant adds contributions at {extra[:3]}")
        n_hidden += int(sum(sb["weight"])) - int(sum(s["weight"]))
    # the step: far-wall cells near the step are hidden (some, not all)
    step, vs, tr = cases[0]
    o = oracle.Oracle(vs, tr, 1 << 20, library=lib, reproject=True)
    o.integrate(step)
    b = oracle.Oracle(vs, tr, 1 << 20, library=lib)
    b.integrate(step)
    lost = b.totals()["voxel_updates"] - o.totals()["voxel_updates"]
    if not 0 < lost < b.totals()["voxel_updates"] // 4:
        f.append(f"step frame: {lost} of {b.totals()['voxel_updates']} contributions hidden")
    # the fronto-parallel plane: nothing is hidden
    plane = scenes.plane_frame()
    o = oracle.Oracle(0.01, 0.04, 4096, library=lib, reproject=True)
    o.integrate(plane)
    b = oracle.Oracle(0.01, 0.04, 4096, library=lib)
    b.integrate(plane)
    if o.totals() != b.totals():
        f.append("plane: the reprojection variant changed the result")
    if n_hidden == 0:
        f.append("no contribution was hidden: the pin did not exercise the test")
    if n_ties > 0.05 * n_kept:
        f.append(f"{n_ties} tie decisions against {n_kept} contributions")
    return f


def sphere_failures(lib=oracle.LIBRARY, frames=range(10)):
    """Analytic sphere r = 0.5 m at (0, 0, 1.5), noise-free depth: along each
    voxel column near the optical axis the linear zero crossing of the mean
    TSDF lies within a quarter voxel of the sphere surface (the paper's
    analytic gate; a half-voxel bias in where the distance is evaluated shows
    up here as a 5 mm error)."""
    f = []
    wl = scenes.workload("spherewall320x240_noisefree")
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity, library=lib)
    for i in frames:
        o.integrate(wl.frame(i))
    k, s = _voxel_table(o)
    mean = s["tsdf"] / s["weight"]
    vs = wl.voxel_size
    worst = 0.0
    n_cols = 0
    for ix in range(-4, 4):
        for iy in range(-4, 4):
            sel = (k[:, 0] == ix) & (k[:, 1] == iy) & (k[:, 2] < 120)
            kz = k[sel, 2]
            m = mean[sel]
            order = np.argsort(kz)
            kz, m = kz[order], m[order]
            cross = None
            for j in range(len(kz) - 1):
                if kz[j + 1] == kz[j] + 1 and m[j] > 0 >= m[j + 1]:
                    z0 = (kz[j] + 0.5) * vs
                    cross = z0 + vs * m[j] / (m[j] - m[j + 1])
                    break
            if cross is None:
                f.append(f"no zero crossing in column ({ix},{iy})")
                continue
            xc, yc = (ix + 0.5) * vs, (iy + 0.5) * vs
            surface = 1.5 - math.sqrt(0.25 - xc * xc - yc * yc)
            worst = max(worst, abs(cross - surface))
            n_cols += 1
    if not worst <= vs / 4:
        f.append(f"sphere zero crossing off by {worst * 1000:.3f} mm (> {vs / 4 * 1000:.2f} mm)")
    if n_cols < 60:
        f.append(f"only {n_cols} columns")
    return f


def invariant_failures(lib=oracle.LIBRARY):
    """Order independence (sums commute), exact pool-exhaustion accounting,
    re-integration, value ranges and count consistency."""
    f = []
    wl = scenes.workload("spherewall320x240")
    frames = [wl.frame(i) for i in (0, 4, 9)]
    vs, tr = wl.voxel_size, wl.trunc

    a = oracle.Oracle(vs, tr, 1 << 20, track_touched=True, library=lib)
    st0 = a.integrate(frames[0])
    ka, sa = _voxel_table(a)
    if st0["voxels_touched"] != len(ka):
        f.append("U != voxels with weight after one frame")
    if st0["blocks_touched"] != a.block_count() or st0["blocks_new"] != a.block_count():
        f.append("B_t / B_n != blocks after one frame")
    for fr in frames[1:]:
        a.integrate(fr)
    b = oracle.Oracle(vs, tr, 1 << 20, library=lib)
    for fr in (frames[2], frames[0], frames[1]):
        b.integrate(fr)
    ca, cb = a.block_coords(), b.block_coords()
    if not np.array_equal(ca, cb):
        f.append("block set depends on frame order")
    else:
        sa, sb = a.block_sums(ca), b.block_sums(cb)
        if not np.array_equal(sa["weight"], sb["weight"]):
            f.append("weights depend on frame order")
        for n in ("tsdf", "r", "g", "b"):
            if not np.allclose(sa[n], sb[n], rtol=0, atol=1e-9):
                f.append(f"{n} sums depend on frame order")
        w = sa["weight"]
        if np.any(w.max(1) <= 0):
            f.append("a block without any contribution")
        tot = a.totals()
        if int(w.sum()) != tot["voxel_updates"]:
            f.append("sum of weights != voxel updates")
        m = w > 0
        mt = sa["tsdf"][m] / w[m]
        if mt.min() < -1 - 1e-12 or mt.max() > 1 + 1e-12:
            f.append("mean TSDF outside [-1, 1]")
        for n in ("r", "g", "b"):
            mc = sa[n][m] / w[m]
            if mc.min() < 0 or mc.max() > 1 + 1e-12:
                f.append(f"mean {n} outside [0, 1]")

    # pool exhaustion: exactly N - cap keys refused, misses account for the rest
    n_blocks = a.block_count()
    cap = n_blocks - 7
    c = oracle.Oracle(vs, tr, cap, library=lib)
    for fr in frames:
        c.integrate(fr)
    tc = c.totals()
    if tc["blocks"] != cap or tc["pool_overflow"] != 7:
        f.append(f"exhaustion: blocks {tc['blocks']} overflow {tc['pool_overflow']} (want {cap}, 7)")
    wc = c.block_sums(c.block_coords())["weight"]
    if int(wc.sum()) + tc["update_misses"] != tc["voxel_updates"]:
        f.append("exhaustion: weights + misses != voxel updates")
    if tc["voxel_updates"] != a.totals()["voxel_updates"]:
        f.append("exhaustion changed the voxel-update count")

    # the same frame twice: no new blocks, weights double
    d = oracle.Oracle(vs, tr, 1 << 20, library=lib)
    d.integrate(frames[0])
    w1 = d.block_sums(d.block_coords())["weight"].copy()
    st = d.integrate(frames[0])
    w2 = d.block_sums(d.block_coords())["weight"]
    if st["blocks_new"] != 0 or not np.array_equal(w2, 2 * w1):
        f.append("re-integrating a frame changed the block set or did not double weights")
    return f


def _weighted_voxels(o):
    """Set of global voxel indices with weight > 0, and the block set."""
    coords = o.block_coords()
    k, _ = _voxel_table(o, coords)
    return {tuple(int(x) for x in kk) for kk in k}, {tuple(int(x) for x in c) for c in coords}


def counter_failures(lib=oracle.LIBRARY):
    """The measurement counts the benchmark divides by, pinned to independent
    recounts: cells visited per point equals the number of cells a
    float64 brute force finds the band segment crossing (tie-free points);
    over an overlapping frame sequence, each frame's distinct blocks B_t and
    distinct voxels U equal the block count and weighted-voxel count of that
    frame integrated alone into a fresh volume, and its new blocks B_n the
    growth of the block count; per call (several frames counted as one
    batch) the distinct blocks, the new blocks and the distinct voxels split
    into those of blocks the call created and of older blocks equal the same
    recounts over the call's frames."""
    f = []
    # cells visited, point by point and per frame
    n_checked = 0
    for frame, vs, tr in _bf_cases():
        H, W = frame.depth.shape
        depth = frame.depth.copy()
        want_frame = 0
        for v in range(H):
            for u in range(W):
                n, tie = bruteforce.crossed_cells(frame, u, v, vs, tr)
                if n is None:
                    continue
                if tie:
                    depth[v, u] = 0.0
                    continue
                o = oracle.Oracle(vs, tr, 1 << 20, library=lib)
                st = o.integrate(_single_pixel(frame, u, v))
                if st["cells_visited"] != n:
                    f.append(f"point ({u},{v}) vs={vs}: {st['cells_visited']} cells visited, brute force {n}")
                    if len(f) > 5:
                        return f
                want_frame += n
                n_checked += 1
        fr = scenes.Frame(depth, frame.rgb, frame.fx, frame.fy, frame.cx, frame.cy, frame.R, frame.t)
        st = oracle.Oracle(vs, tr, 1 << 20, library=lib).integrate(fr)
        if st["cells_visited"] != want_frame:
            f.append(f"frame vs={vs}: {st['cells_visited']} cells visited, brute force {want_frame}")
    if n_checked < 150:
        f.append(f"only {n_checked} points with a cell count")

    # per frame: B_t, U, B_n over an overlapping sequence
    wl = scenes.workload("spherewall320x240")
    frames = [wl.frame(i) for i in (0, 4, 9, 4)]
    vs, tr = wl.voxel_size, wl.trunc
    a = oracle.Oracle(vs, tr, 1 << 20, track_touched=True, library=lib)
    for i, fr in enumerate(frames):
        before = a.block_count()
        st = a.integrate(fr)
        alone = oracle.Oracle(vs, tr, 1 << 20, library=lib)
        alone.integrate(fr)
        vox, blocks = _weighted_voxels(alone)
        if st["blocks_touched"] != len(blocks):
            f.append(f"frame {i}: B_t {st['blocks_touched']} != {len(blocks)} blocks of the frame alone")
        if st["voxels_touched"] != len(vox):
            f.append(f"frame {i}: U {st['voxels_touched']} != {len(vox)} weighted voxels of the frame alone")
        if st["blocks_new"] != a.block_count() - before:
            f.append(f"frame {i}: B_n {st['blocks_new']} != growth {a.block_count() - before}")
    # per call: two calls of two frames each, the second overlapping the first
    calls = [[frames[0], frames[1]], [frames[2], frames[1]]]
    c = oracle.Oracle(vs, tr, 1 << 20, track_touched=True, library=lib)
    prev_blocks = set()
    for j, call in enumerate(calls):
        if j:
            c.begin_call()
        before = c.block_count()
        for fr in call:
            c.integrate(fr)
        cs = c.call_stats()
        alone = oracle.Oracle(vs, tr, 1 << 20, library=lib)
        for fr in call:
            alone.integrate(fr)
        vox, blocks = _weighted_voxels(alone)
        fresh = {k for k in vox if tuple(x // 8 for x in k) not in prev_blocks}
        want = {"frames": len(call), "blocks_touched": len(blocks), "blocks_new": c.block_count() - before,
                "voxels_fresh": len(fresh), "voxels_old": len(vox) - len(fresh)}
        if cs != want:
            f.append(f"call {j}: counts {cs} != recount {want}")
        _, prev_blocks = _weighted_voxels(c)
    if calls and not want["voxels_old"]:
        f.append("the second call touched no older voxel: the pin did not exercise the split")
    return f


def edge_failures(lib=oracle.LIBRARY):
    """Empty, invalid, near and out-of-range inputs."""
    f = []
    base = scenes.random_frame(11, W=9, H=6)
    vs, tr = 0.01, 0.04

    def run(depth, t=None):
        o = oracle.Oracle(vs, tr, 1 << 16, library=lib)
        fr = scenes.Frame(np.ascontiguousarray(depth, np.float32), base.rgb[: depth.shape[0], : depth.shape[1]]
                          if depth.size else np.zeros(depth.shape + (3,), np.uint8),
                          base.fx, base.fy, base.cx, base.cy, base.R,
                          base.t if t is None else np.asarray(t, np.float32))
        return o.integrate(fr), o

    st, o = run(np.zeros((6, 9)))
    if st["points_valid"] or o.block_count():
        f.append("all-zero frame produced points")
    st, o = run(np.zeros((0, 0)))
    if st["points_valid"] or o.block_count():
        f.append("empty frame produced points")
    d = np.full((6, 9), np.nan)
    d[0, :3] = [np.inf, -np.inf, -1.0]
    st, o = run(d)
    if st["points_valid"] or st["near_skipped"] or o.block_count():
        f.append("non-finite / negative depths were used")
    d = np.full((6, 9), 0.03)              # 0 < d <= trunc
    d[1, 1] = tr
    st, o = run(d)
    if st["near_skipped"] != 54 or st["points_valid"]:
        f.append(f"near points: {st['near_skipped']} skipped")
    st, o = run(base.depth, t=[1e5, 0.0, 0.0])   # 10^7 voxels from the origin
    if st["out_of_range"] != 54 or st["points_valid"] or o.block_count():
        f.append(f"out of range: {st['out_of_range']}")
    st, o = run(base.depth, t=[80000.0, 0.0, 0.0])  # inside the key range
    if st["out_of_range"] or st["points_valid"] != 54:
        f.append("in-range far points rejected")
    return f


# ---------------------------------------------------------------------------
# surface extraction (marching tetrahedra, mesh_oracle.cpp)
# ---------------------------------------------------------------------------
def _field_volume(nb, vs, value, observed=None, origin=(-2, -2, -2)):
    """Blocks origin + [0, nb)^3 with the sums of a field sampled at voxel
    centres: tsdf = value(centres) (weight 1) where observed."""
    o = np.asarray(origin)
    coords = np.array([[x, y, z] for x in range(nb) for y in range(nb) for z in range(nb)], np.int32) + o
    li = np.arange(512)
    local = np.stack([li % 8, (li // 8) % 8, li // 64], 1)
    k = coords[:, None, :].astype(np.int64) * 8 + local[None]
    centres = (k + 0.5) * vs
    w = np.ones(k.shape[:2]) if observed is None else observed(k).astype(np.float64)
    t = value(centres) * w
    return coords, t, w


def _mesh_edges(tris):
    """Directed edges (a, b) of every triangle, as an (3 nt, 2) array."""
    return np.concatenate([tris[:, [0, 1]], tris[:, [1, 2]], tris[:, [2, 0]]])


def _orientation_failures(m, label, closed):
    """Every undirected edge is used by at most two triangles (exactly two if
    the surface is closed), and two triangles sharing an edge run it in
    opposite directions (a consistently oriented surface)."""
    f = []
    e = _mesh_edges(m.tris)
    und = np.sort(e, 1)
    _, inv, cnt = np.unique(und, axis=0, return_inverse=True, return_counts=True)
    if cnt.max(initial=0) > 2:
        f.append(f"{label}: an edge shared by {cnt.max()} triangles")
    if closed and cnt.min(initial=2) != 2:
        f.append(f"{label}: {int((cnt != 2).sum())} edges not shared by exactly two triangles (not closed)")
    directed, dcnt = np.unique(e, axis=0, return_counts=True)
    if dcnt.max(initial=0) > 1:
        f.append(f"{label}: a directed edge used twice (inconsistent orientation)")
    return f


def _normals(m):
    a, b, c = (m.pos[m.tris[:, i]] for i in range(3))
    return np.cross(b - a, c - a), (a + b + c) / 3.0


def mesh_field_failures(lib=oracle.MESH_LIBRARY):
    """Extraction on fields sampled at voxel centres (no integration): a
    linear field's vertices lie exactly on its zero plane and its triangles
    face along the gradient; a sphere's signed distance, observed in a box
    around it, gives a closed, consistently oriented surface with Euler
    characteristic 2, outward normals and vertices on the sphere; a random
    field gives a consistently oriented manifold; no vertex sits on an edge
    with an unobserved end."""
    f = []
    vs = 0.02
    rng = np.random.default_rng(31)
    # linear fields: linear interpolation of a linear function is exact
    for trial in range(3):
        n = rng.normal(size=3)
        n /= np.linalg.norm(n)
        c = float(rng.uniform(-0.05, 0.05))
        coords, t, w = _field_volume(4, vs, lambda x: (x @ n - c) / (4 * vs))
        m = oracle.extract_mesh(coords, t, w, vs, library=lib)
        if len(m.tris) < 100:
            f.append(f"plane field {trial}: only {len(m.tris)} triangles")
            continue
        err = np.abs(m.pos @ n - c).max()
        if not err < 1e-12:
            f.append(f"plane field {trial}: a vertex {err:.3g} m off the plane")
        nrm, _ = _normals(m)
        if np.any(nrm @ n < -1e-15):
            f.append(f"plane field {trial}: a triangle faces against the gradient")
        f += _orientation_failures(m, f"plane field {trial}", closed=False)
    # a sphere's signed distance (truncated), observed in a 0.64 m box
    centre, r = np.array([0.013, -0.021, 0.007]), 0.2
    trunc = 4 * vs
    coords, t, w = _field_volume(4, vs, lambda x: np.clip((np.linalg.norm(x - centre, axis=-1) - r) / trunc, -1, 1))
    m = oracle.extract_mesh(coords, t, w, vs, library=lib)
    f += _orientation_failures(m, "sphere field", closed=True)
    V, F = len(m.pos), len(m.tris)
    E = len(np.unique(np.sort(_mesh_edges(m.tris), 1), axis=0))
    if V - E + F != 2:
        f.append(f"sphere field: Euler characteristic {V - E + F} != 2")
    d = np.linalg.norm(m.pos - centre, axis=1) - r
    if not np.abs(d).max() <= vs / 4:
        f.append(f"sphere field: a vertex {np.abs(d).max() * 1000:.3f} mm off the sphere")
    nrm, cen = _normals(m)
    if np.any(np.einsum("ij,ij->i", nrm, cen - centre) <= 0):
        f.append("sphere field: a triangle faces inwards")
    # a random field over a region with unobserved voxels
    vals = rng.uniform(-1, 1, size=(64, 512))
    obs = rng.random((64, 512)) > 0.1
    coords = np.array([[x, y, z] for x in range(4) for y in range(4) for z in range(4)], np.int32) - 2
    m = oracle.extract_mesh(coords, vals * obs, obs.astype(np.float64), vs, library=lib)
    f += _orientation_failures(m, "random field", closed=False)
    li = np.arange(512)
    observed = {tuple(int(x) for x in cc * 8 + np.array([l % 8, (l // 8) % 8, l // 64]))
                for b, cc in enumerate(coords) for l in li[obs[b]]}
    ends = [(tuple(int(x) for x in k[:3]), tuple(int(k[i]) + ((int(k[3]) >> i) & 1) for i in range(3)))
            for k in m.keys]
    if any(a not in observed or b not in observed for a, b in ends):
        f.append("random field: a vertex on an edge with an unobserved end")
    if len(m.tris) < 1000:
        f.append(f"random field: only {len(m.tris)} triangles")
    # the vertex key names a lattice edge whose ends straddle the surface
    sums = {}
    for b, cc in enumerate(coords):
        for l in range(512):
            sums[tuple(int(x) for x in cc * 8 + np.array([l % 8, (l // 8) % 8, l // 64]))] = vals[b, l] * obs[b, l]
    if any((sums[a] < 0) == (sums[b] < 0) for a, b in ends):
        f.append("random field: a vertex on an edge whose ends lie on the same side")
    return f


def _dense_plane():
    """The plane workload's geometry (z = 1 m, identity pose) seen with 5 mm
    pixels at 1 m, finer than the 1 cm voxels: every voxel column of the
    view is observed."""
    return scenes.plane_frame(W=160, H=120, fx=200.0, fy=200.0, cx=79.5, cy=59.5)


def mesh_plane_failures(lib=oracle.MESH_LIBRARY):
    """Integration and extraction of a fronto-parallel plane at z = 1 m
    (vs 1 cm, trunc 4 cm): every voxel of layer 99 holds +0.125 and of layer
    100 -0.125, so every vertex lies at z = 1.000 m, only on edges from layer
    99 to layer 100; every cell of those layers with eight observed corners
    holds exactly 8 triangles covering its cross-section, area vs^2, each
    facing the camera (-z: from behind the surface to in front of it)."""
    f = []
    vs, tr = 0.01, 0.04
    o = oracle.Oracle(vs, tr, 1 << 16)
    o.integrate(_dense_plane())
    coords = o.block_coords()
    s = o.block_sums(coords)
    m = oracle.extract_mesh(coords, s["tsdf"], s["weight"], vs, library=lib)
    if len(m.tris) < 1000:
        return [f"dense plane: only {len(m.tris)} triangles"]
    if not np.abs(m.pos[:, 2] - 1.0).max() < 1e-6:
        f.append(f"dense plane: a vertex at z = {m.pos[np.argmax(np.abs(m.pos[:, 2] - 1.0)), 2]:.7f}")
    if not (np.all(m.keys[:, 2] == 99) and np.all(m.keys[:, 3] & 4)):
        f.append("dense plane: a vertex on an edge that is not from layer 99 to layer 100")
    k, _ = _voxel_table(o, coords)
    obs = {tuple(int(x) for x in kk) for kk in k}
    full = {(i, j) for (i, j, z) in obs if z == 99 and all(
        (i + a, j + b, 99 + c) in obs for a in (0, 1) for b in (0, 1) for c in (0, 1))}
    nrm, cen = _normals(m)
    cell = np.floor(cen[:, :2] / vs - 0.5).astype(np.int64)
    area = 0.5 * np.linalg.norm(nrm, axis=1)
    per = {}
    for (i, j), a in zip(map(tuple, cell.tolist()), area):
        n_, s_ = per.get((i, j), (0, 0.0))
        per[(i, j)] = (n_ + 1, s_ + a)
    bad = [c for c in full if per.get(c, (0, 0.0))[0] != 8 or abs(per[c][1] - vs * vs) > 1e-12]
    if bad:
        f.append(f"dense plane: {len(bad)} of {len(full)} fully observed cells without 8 triangles of area vs^2")
    if len(full) < 3000:
        f.append(f"dense plane: only {len(full)} fully observed cells")
    if np.any(nrm[:, 2] >= 0):
        f.append("dense plane: a triangle faces away from the camera")
    return f


def mesh_sphere_failures(lib=oracle.MESH_LIBRARY):
    """The analytic sphere gate: the noise-free sphere-and-wall sequence
    integrated, then extracted: every vertex on the sphere's front cap (seen
    head-on by the arc of cameras) lies within a quarter voxel of the sphere
    r = 0.5 m at (0, 0, 1.5)."""
    f = []
    wl = scenes.workload("spherewall320x240_noisefree")
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity)
    for i in range(wl.n_frames):
        o.integrate(wl.frame(i))
    coords = o.block_coords()
    s = o.block_sums(coords)
    m = oracle.extract_mesh(coords, s["tsdf"], s["weight"], wl.voxel_size, library=lib)
    cap = (m.pos[:, 2] < 1.2) & (np.hypot(m.pos[:, 0], m.pos[:, 1]) < 0.2)
    if cap.sum() < 500:
        return [f"sphere: only {int(cap.sum())} vertices on the front cap"]
    d = np.abs(np.linalg.norm(m.pos[cap] - np.array([0.0, 0.0, 1.5]), axis=1) - 0.5)
    if not d.max() <= wl.voxel_size / 4:
        f.append(f"sphere: a cap vertex {d.max() * 1000:.3f} mm off the sphere (> {wl.voxel_size / 4 * 1000:.2f} mm)")
    f += _orientation_failures(m, "sphere scene", closed=False)
    return f


PINS = {
    "plane": plane_failures,
    "bruteforce": bruteforce_failures,
    "reprojection": reprojection_failures,
    "sphere": sphere_failures,
    "invariants": invariant_failures,
    "counters": counter_failures,
    "edges": edge_failures,
}
# pins of the extraction oracle (their `lib` is the mesh library)
MESH_PINS = {
    "mesh_fields": mesh_field_failures,
    "mesh_plane": mesh_plane_failures,
    "mesh_sphere": mesh_sphere_failures,
}


if __name__ == "__main__":
    lib_path = sys.argv[1]
    names = sys.argv[2].split(",")
    out = {}
    for n in names:
        try:
            out[n] = {**PINS, **MESH_PINS}[n](lib_path)
        except Exception as e:           # a planted mistake may break a check outright
            out[n] = [f"exception: {type(e).__name__}: {e}"]
    print(json.dumps(out))
