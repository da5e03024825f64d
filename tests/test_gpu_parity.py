"""HIP library vs oracle on the same seeded inputs (needs an MI355X).

Bit-exact: block set, block count, per-voxel weights, point / update / loss
counts.  Within 1e-4: mean TSDF and mean colour.  Workloads: the plane, the
sphere-and-wall arc, the 640 x 480 room (a prefix element by element, and
all 100 frames in the benchmark's launch configuration), the 1280 x 720 room
at its full sizes, the 0.2 m contention cube, the load-factor sweep and the
bounded-probe control on it, tiny random frames with ragged sizes, walks several chunks long, dense
blocks spanning several LDS windows, batches, band ends hit exactly and
far cameras, and the edge cases.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from hash_table_amd import scenes
from tests import parity
from tests.parity import say

pytestmark = pytest.mark.gpu
MODES = ["owner", "rays"]
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, f"{name}_counts.json")) as fh:
        return json.load(fh)


def run_both(frames, vs, tr, cap, table=0, split=False, mode="owner", batch=1, max_batch_pixels=0):
    frames = list(frames)
    say(f"  gpu ({mode}, batch {batch}): {len(frames)} frame(s) {frames[0].width}x{frames[0].height} "
        f"vs={vs} trunc={tr} cap={cap}")
    vol, st, coords, arrays, _ = parity.gpu_integrate(frames, vs, tr, cap, table, split=split, mode=mode,
                                                      batch=batch, max_batch_pixels=max_batch_pixels)
    say(f"  oracle: {len(frames)} frame(s)")
    o = parity.oracle_integrate(frames, vs, tr, cap)
    return vol, st, coords, arrays, o


def assert_parity(st, coords, arrays, o, expect_loss=False):
    f = parity.compare_stats(st, o, expect_loss) + parity.compare_blocks(coords, arrays, o)
    assert f == [], f


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build()


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
def test_plane_parity(mode):
    wl = scenes.workload("plane64x48")
    _, st, coords, arrays, o = run_both([wl.frame(0)], wl.voxel_size, wl.trunc, wl.pool_capacity, mode=mode)
    assert st["pool_used"] == 234
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["spherewall320x240", "spherewall320x240_noisefree"])
def test_sphere_wall_parity(name, mode):
    wl = scenes.workload(name)
    _, st, coords, arrays, o = run_both(wl.frames(), wl.voxel_size, wl.trunc, wl.pool_capacity, mode=mode)
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("name", ["plane64x48", "spherewall320x240", "cube640x480"])
def test_no_rescans_with_record_buffers_sized_for_the_call(name):
    """Record buffers sized for exactly the call's pixels (as the benchmark
    sizes them; small frames fill few of the record partitions, one per
    16 x 16 tile): every run is recorded, no block is rescanned."""
    wl = scenes.workload(name)
    frames = list(wl.frames())
    px = sum(f.width * f.height for f in frames)
    _, st, coords, arrays, o = run_both(frames, wl.voxel_size, wl.trunc, wl.pool_capacity, batch=len(frames),
                                        max_batch_pixels=px)
    assert st["fallback_blocks"] == 0
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
def test_cube_contention_parity(mode):
    wl = scenes.workload("cube640x480")
    _, st, coords, arrays, o = run_both([wl.frame(0)], wl.voxel_size, wl.trunc, wl.pool_capacity, mode=mode)
    assert_parity(st, coords, arrays, o)
    assert st["voxel_updates"] / max(st["pool_used"], 1) > 10000      # heavy same-block contention


@pytest.mark.parametrize("mode", MODES)
def test_room_prefix_parity_split_calls(mode):
    # separate tsdf_allocate / tsdf_update calls, first 6 frames, element by element
    wl = scenes.workload("room640x480")
    _, st, coords, arrays, o = run_both(wl.frames(0, 6), wl.voxel_size, wl.trunc, wl.pool_capacity, split=True,
                                        mode=mode)
    assert_parity(st, coords, arrays, o)


def _check_history(label, hist, g, calls):
    """Per-call counters against the oracle's stored per-frame counts."""
    for h, c in zip(hist, calls):
        last = c[-1]
        assert h["pool_used"] == g["frames"][last]["blocks_total"], f"{label} after frame {last}: blocks"
        assert h["voxel_updates"] == sum(f["voxel_updates"] for f in g["frames"][:last + 1]), \
            f"{label} after frame {last}: voxel updates"
        assert h["points_valid"] == sum(f["points_valid"] for f in g["frames"][:last + 1]), \
            f"{label} after frame {last}: valid points"


@pytest.mark.timeout(600)
def test_room_full_parity():
    """All 100 frames of the 640 x 480 room: in the launch configuration the
    benchmark times (owner update, all 100 frames in one call) and one frame
    per call with both update modes; counts after every call against the
    stored oracle counts, then every voxel against a live oracle run."""
    wl = scenes.workload("room640x480")
    g = golden("room640x480")
    frames = list(wl.frames())
    for i, f in enumerate(frames[:3]):
        assert scenes.frame_digest([f]) == g["frames"][i]["sha256"], "generator drifted from the stored counts"
    results = {}
    for mode, batch in (("owner", 100), ("owner", 1), ("rays", 1)):
        say(f"  gpu ({mode}, {batch} frames per call): 100 frames 640x480")
        _, st, coords, arrays, hist = parity.gpu_integrate(frames, wl.voxel_size, wl.trunc, wl.pool_capacity,
                                                           per_frame_stats=True, mode=mode, batch=batch,
                                                           max_batch_pixels=batch * 640 * 480)
        calls = [list(range(i, min(i + batch, 100))) for i in range(0, 100, batch)]
        _check_history(f"{mode}/{batch}", hist, g, calls)
        assert st["fallback_blocks"] == 0
        results[(mode, batch)] = (st, coords, arrays)
    say("  oracle: 100 frames")
    o = parity.oracle_integrate(frames, wl.voxel_size, wl.trunc, wl.pool_capacity)
    for key, (st, coords, arrays) in results.items():
        say(f"  compare {key}")
        err = {}
        f = parity.compare_stats(st, o) + parity.compare_blocks(coords, arrays, o, errors=err)
        say(f"    largest mean differences: " + ", ".join(f"{k} {v:.3g}" for k, v in err.items()))
        assert f == [], f
        if key == ("owner", 100):
            # one call: each block's sums are added in LDS (signed distance
            # in 2^-24 units) and written once, so a mean differs from the
            # oracle's by float rounding only, far inside 1e-4
            assert max(err.values()) <= 2.0 ** -20, err


@pytest.mark.timeout(1200)
def test_room1280x720_full_sequence():
    """The 1280 x 720 room at its full sizes and length -- 300 frames of
    921,600 pixels, a pool of 2^22 blocks (40 GiB of sums), a 2^24-entry
    table -- in the benchmark's launch configuration (owner update, calls of
    100 frames): counts after every call against the stored oracle counts,
    then the block set in full and every voxel's weight and means against the
    oracle run over all 300 frames (in eight worker processes, each over a
    contiguous range of frames, their sums added)."""
    wl = scenes.workload("room1280x720")
    g = golden("room1280x720")
    n, batch = wl.n_frames, 100
    say(f"  oracle and frames: {n} frames 1280x720 in 8 worker processes")
    frames, o = parity.oracle_ranges("room1280x720", n, workers=8)
    for i in (0, n // 2, n - 1):
        assert scenes.frame_digest([frames[i]]) == g["frames"][i]["sha256"], "generator drifted"
    assert o.block_count() == g["frames"][-1]["blocks_total"]
    assert o.totals()["voxel_updates"] == g["totals"]["voxel_updates"]
    say(f"  gpu: {n} frames, pool {wl.pool_capacity}, table {wl.table_entries}, {batch} frames per call")
    vol, st, coords, arrays, hist = parity.gpu_integrate(frames, wl.voxel_size, wl.trunc, wl.pool_capacity,
                                                         wl.table_entries, per_frame_stats=True, batch=batch,
                                                         max_batch_pixels=batch * wl.width * wl.height)
    _check_history("1280x720", hist, g, [list(range(i, min(i + batch, n))) for i in range(0, n, batch)])
    assert st["fallback_blocks"] == 0
    del frames
    say(f"  compare {len(coords)} blocks voxel by voxel")
    err = {}
    f = parity.compare_stats(st, o) + parity.compare_blocks(coords, arrays, o, errors=err)
    say(f"    largest mean differences: " + ", ".join(f"{k} {v:.3g}" for k, v in err.items()))
    assert f == [], f
    table = vol.table.view(-1, 2).cpu().numpy().view(np.uint64)
    f = parity.table_layout_failures(table, o.block_coords(), wl.pool_capacity)
    assert f == [], f


@pytest.mark.timeout(900)
def test_sweep_cells():
    """The benchmark's sweep cells (the room scene at 160x120 ... 1280x960,
    along the point-count and extent axes), 16 frames in one batched call:
    counts against the oracle's stored counts, and every voxel against a live
    oracle run, for every cell."""
    for axis, W, H, fx in scenes.SWEEP_CELLS:
        name = scenes.cell_name(W, H, fx) if (W, H, fx) != (640, 480, 525.0) else "room640x480"
        wl = scenes.workload(name)
        g = golden(name)
        frames = list(wl.frames(0, 16))
        assert scenes.frame_digest([frames[15]]) == g["frames"][15]["sha256"], "generator drifted"
        say(f"  {axis} cell {name}")
        _, st, coords, arrays, _ = parity.gpu_integrate(frames, wl.voxel_size, wl.trunc, wl.pool_capacity,
                                                        batch=16, max_batch_pixels=16 * W * H)
        assert st["pool_used"] == g["frames"][15]["blocks_total"]
        assert st["voxel_updates"] == sum(f["voxel_updates"] for f in g["frames"][:16])
        assert st["points_valid"] == sum(f["points_valid"] for f in g["frames"][:16])
        assert st["fallback_blocks"] == 0 and st["update_misses"] == 0 and st["table_full"] == 0
        o = parity.oracle_integrate(frames, wl.voxel_size, wl.trunc, wl.pool_capacity)
        assert_parity(st, coords, arrays, o)


def _reproject_cases():
    from tests import oracle_pins
    cases = [("step", [oracle_pins._step_frame()], 0.2, 0.7, 1 << 16)]
    for seed in (11, 12):
        cases.append((f"random{seed}", [scenes.random_frame(seed, W=37, H=23, translation_scale=0.5)],
                      0.013, 0.052, 1 << 18))
    wl = scenes.workload("spherewall320x240")
    cases.append(("spherewall", list(wl.frames()), wl.voxel_size, wl.trunc, wl.pool_capacity))
    wl = scenes.workload("room640x480")
    cases.append(("room16", list(wl.frames(0, 16)), wl.voxel_size, wl.trunc, wl.pool_capacity))
    cases.append(("room40", list(wl.frames(0, 40)), wl.voxel_size, wl.trunc, wl.pool_capacity))
    return cases


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", MODES)
def test_reprojection_occlusion_parity(mode):
    """The reprojection reading of the occlusion test (the centre also hidden
    behind the depth seen at its own pixel) in both passes: block set,
    weights exact and means within 1e-4 against the oracle with the same
    reading, one frame per call and 16 per call (40 frames: one call, frames
    32.. from the device frame table); on the scenes with depth
    discontinuities it must hide contributions the projective reading keeps."""
    for name, frames, vs, tr, cap in _reproject_cases():
        for batch in ((40,) if len(frames) > 32 else (1, 16)):
            if batch > 1 and len(frames) == 1:
                continue
            W, H = frames[0].width, frames[0].height
            say(f"  {mode} {name} batch {batch}: {len(frames)} frame(s) {W}x{H}")
            _, st, coords, arrays, _ = parity.gpu_integrate(frames, vs, tr, cap, mode=mode, batch=batch,
                                                            max_batch_pixels=batch * W * H, occlusion="reproject")
            o = parity.oracle_integrate(frames, vs, tr, cap, reproject=True)
            assert_parity(st, coords, arrays, o)
        base = parity.oracle_integrate(frames, vs, tr, cap).totals()["voxel_updates"]
        say(f"    hidden by the image: {base - st['voxel_updates']} of {base}")
        if name in ("step", "spherewall", "room16", "room40"):
            assert st["voxel_updates"] < base


def _lf_case(target):
    """Pool 2^k (table 2^(k+1)) and the longest frame prefix of the room whose
    block count stays within target * table entries."""
    g = golden("room640x480")
    return scenes.load_factor_cell([f["blocks_total"] for f in g["frames"]], target)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("target", [0.1, 0.25, 0.5])
def test_load_factor_parity(target, mode):
    cap, n, lf = _lf_case(target)
    say(f"  load factor target {target}: pool {cap}, table {2 * cap}, {n} frames, achieved {lf:.3f}")
    assert target - 0.1 < lf <= target
    wl = scenes.workload("room640x480")
    vol, st, coords, arrays, o = run_both(wl.frames(0, n), wl.voxel_size, wl.trunc, cap, 2 * cap, mode=mode)
    assert_parity(st, coords, arrays, o)
    # the table itself: the slots linear probing fills, and the total
    # displacement, do not depend on the insertion order (exact)
    table = vol.table.view(-1, 2).cpu().numpy().view(np.uint64)
    f = parity.table_layout_failures(table, o.block_coords(), cap)
    assert f == [], f
    bins = np.arange(1, tsdf_bins() + 1)
    ha = st["probe_hist_alloc"]
    mean_a = float((ha * bins).sum() / ha.sum())
    # the histogram counts every probe sequence (one per distinct key and
    # workgroup filing): at least one slot each, and at most the longest sequence
    # the final layout allows
    disp = table_displacements(table, o.block_coords())
    say(f"  allocate probes: mean {mean_a:.3f} (Knuth's insertion expectation "
        f"{0.5 * (1 + 1 / (1 - lf) ** 2):.3f}), max {st['probe_max']}, longest final displacement {disp.max()}")
    assert ha.sum() > 0 and mean_a >= 1.0
    assert st["probe_max"] <= disp.max() + 1
    if mode == "rays":
        # lookups after allocation: near the successful-search expectation
        h = st["probe_hist_update"]
        mean = float((h * bins).sum() / h.sum())
        knuth = 0.5 * (1 + 1 / (1 - lf))
        say(f"  update probes: mean {mean:.3f}, Knuth {knuth:.3f}")
        assert abs(mean - knuth) < 0.35 * knuth


@pytest.mark.parametrize("mode", MODES)
def test_bounded_probe_control_counts_every_loss(mode):
    # The paper's section 7: a probe bounded at 8 slots (its Triton arm) loses
    # blocks once the table fills, silently there.  The same bound here (a
    # negative control, never the default) must lose only whole keys -- every
    # surviving block exact -- and count every lost contribution.
    from hash_table_amd import tsdf
    wl = scenes.workload("room640x480")
    lost_any = False
    for target in (0.1, 0.25, 0.5):
        cap, n, lf = _lf_case(target)
        frames = list(wl.frames(0, n))
        vol = tsdf.Volume(wl.voxel_size, wl.trunc, cap, 2 * cap, update_mode=mode, probe_limit=8)
        for i in range(0, n, 16):
            vol.integrate_batch([tsdf.DeviceFrame(f) for f in frames[i:i + 16]])
        st = vol.stats()
        coords, arrays = vol.export()
        o = parity.oracle_integrate(frames, wl.voxel_size, wl.trunc, cap)
        tot = o.totals()
        oc = {tuple(c) for c in o.block_coords().tolist()}
        gc = {tuple(c) for c in coords.tolist()}
        lost = oc - gc
        say(f"  {mode} load factor {lf:.3f} ({n} frames): blocks {len(gc)} of {len(oc)}, "
            f"probe_exhausted {st['probe_exhausted']}, update_misses {st['update_misses']}, probe_max {st['probe_max']}")
        assert gc <= oc and st["probe_max"] <= 8
        assert st["voxel_updates"] == tot["voxel_updates"] and st["table_full"] == 0
        if lost:
            lost_any = True
            assert st["probe_exhausted"] >= len(lost)
        w_lost = float(o.block_sums(np.array(sorted(lost), np.int32).reshape(-1, 3))["weight"].sum()) if lost else 0.0
        assert st["update_misses"] == w_lost                     # every lost contribution counted
        assert float(arrays["weight"].astype(np.float64).sum()) + st["update_misses"] == tot["voxel_updates"]
        f = parity.compare_blocks(coords, arrays, _OracleSubset(o, gc))
        assert f == [], f                                        # surviving blocks are exact
        del vol
    assert lost_any, "the bounded probe never ran out: the control did not exercise the loss"


class _OracleSubset:
    """An oracle view restricted to the blocks the GPU kept (for comparing
    the survivors of the bounded-probe control)."""

    def __init__(self, o, keep):
        self.o, self.keep = o, keep

    def block_coords(self):
        c = self.o.block_coords()
        m = np.array([tuple(x) in self.keep for x in c.tolist()], bool)
        return c[m]

    def block_sums(self, coords):
        return self.o.block_sums(coords)


def table_displacements(table, coords):
    """Slots past its home slot of every key, from an exported table."""
    T = table.shape[0]
    tk = table[:, 0]
    occ = np.nonzero(tk != np.uint64(0xFFFFFFFFFFFFFFFF))[0]
    where = {int(k): int(i) for k, i in zip(tk[occ].tolist(), occ.tolist())}
    keys = parity._pack(coords).astype(np.uint64)
    home = (parity.fmix64(keys) & np.uint64(T - 1)).astype(np.int64)
    pos = np.array([where[int(k)] for k in keys.tolist()], np.int64)
    return (pos - home) & (T - 1)


def tsdf_bins():
    from hash_table_amd import tsdf
    return tsdf.TSDF_PROBE_BINS


# ---------------------------------------------------------------------------
# batched integration (one allocate and one update for several frames)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("batch", [3, 16, 40])
def test_batched_room_parity(mode, batch):
    # 40: one call whose frames 32.. travel in the device frame table and
    # whose run records carry the frame's high bits
    wl = scenes.workload("room640x480")
    frames = list(wl.frames(0, max(20, batch)))
    _, st, coords, arrays, o = run_both(frames, wl.voxel_size, wl.trunc, wl.pool_capacity, mode=mode,
                                        batch=batch, max_batch_pixels=batch * 640 * 480)
    assert_parity(st, coords, arrays, o)
    assert st["fallback_blocks"] == 0


@pytest.mark.parametrize("mode", MODES)
def test_batch_of_mixed_frames(mode):
    frames = [scenes.random_frame(s, W=W, H=H, invalid_frac=0.1, translation_scale=0.3)
              for s, (W, H) in enumerate([(37, 23), (16, 16), (129, 65), (1, 33), (64, 48)])]
    frames.append(scenes.workload("plane64x48").frame(0))
    _, st, coords, arrays, o = run_both(frames, 0.01, 0.04, 1 << 16, mode=mode, batch=len(frames))
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
def test_full_batch_of_mixed_frames(mode):
    # TSDF_MAX_BATCH frames in one call: sizes from 1 x 1 to 129 x 65, some
    # empty (skipped, so a frame's place in the batch and in the call's
    # frame table differ), poses all different: frames past the first 32
    # travel in the device frame table and their records carry the frame's
    # high bits
    from hash_table_amd import tsdf
    rng = np.random.default_rng(7)
    sizes = [(1, 1), (37, 23), (16, 16), (129, 65), (1, 33), (64, 48), (9, 6)]
    frames = []
    for i in range(tsdf.TSDF_MAX_BATCH):
        W, H = sizes[int(rng.integers(len(sizes)))]
        fr = scenes.random_frame(100 + i, W=W, H=H, invalid_frac=0.1, translation_scale=0.3)
        frames.append(_frame_like(fr, np.zeros((0, 0))) if i % 17 == 5 else fr)
    _, st, coords, arrays, o = run_both(frames, 0.01, 0.04, 1 << 18, mode=mode, batch=len(frames),
                                        max_batch_pixels=sum(f.width * f.height for f in frames))
    assert st["fallback_blocks"] == 0          # the frames' runs spread over the record partitions
    assert_parity(st, coords, arrays, o)


def test_record_overflow_rescans_exactly():
    # run records sized for 2,000 pixels per call: most blocks cannot keep
    # their runs and are rescanned from their pixel rectangles instead
    wl = scenes.workload("spherewall320x240")
    frames = list(wl.frames(0, 4))
    _, st, coords, arrays, o = run_both(frames, wl.voxel_size, wl.trunc, wl.pool_capacity, mode="owner",
                                        batch=2, max_batch_pixels=2000)
    assert st["fallback_blocks"] > 0
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
def test_dense_blocks_span_several_segment_windows(mode):
    # planes 0.1 m in front of a 640 x 480 camera: a 4 cm block covers about
    # 210 x 210 pixels, so one block gathers ~44,000 runs from ~700 wavefront
    # segments per frame -- more than one LDS window of segments, many
    # staged sub-batches of runs and more than one 8191-run pass of packed
    # sums in the owner update
    frames = [scenes.plane_frame(seed=s, W=640, H=480, depth=d, fx=525.0, fy=525.0, cx=319.5, cy=239.5)
              for s, d in ((3, 0.1), (4, 0.1037))]
    _, st, coords, arrays, o = run_both(frames, 0.005, 0.02, 4096, mode=mode, batch=2)
    assert st["fallback_blocks"] == 0
    assert_parity(st, coords, arrays, o)


def test_batch_limits():
    from hash_table_amd import tsdf
    wl = scenes.workload("plane64x48")
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity)
    f = tsdf.DeviceFrame(wl.frame(0))
    with pytest.raises(tsdf.TsdfError):
        vol.integrate_batch([f] * (tsdf.TSDF_MAX_BATCH + 1))
    tsdf.tsdf_integrate_batch(vol.handle, [])          # nothing to do
    vol.integrate_batch([f] * tsdf.TSDF_MAX_BATCH)
    st = vol.stats()
    assert st["pool_used"] == 234 and st["voxel_updates"] == tsdf.TSDF_MAX_BATCH * 38688
    c, a = vol.export()
    assert float(a["weight"].sum()) == tsdf.TSDF_MAX_BATCH * 38688


# ---------------------------------------------------------------------------
# tiny and ragged inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("seed,W,H", [(0, 7, 5), (1, 37, 23), (2, 16, 16), (3, 17, 1), (4, 1, 33), (5, 129, 65)])
def test_random_frames_parity(seed, W, H, mode):
    frames = [scenes.random_frame(seed * 10 + j, W=W, H=H, invalid_frac=0.2, translation_scale=0.3)
              for j in range(3)]
    for vs, tr in ((0.01, 0.04), (0.013, 0.05)):
        _, st, coords, arrays, o = run_both(frames, vs, tr, 1 << 16, mode=mode)
        assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
def test_filing_with_many_distinct_blocks(mode):
    """Wide-angle rays at random depths 1-10 m: the rays of one 16 x 16 tile
    cross ~900 distinct blocks, so a single workgroup filing holds far more
    than 256 distinct keys (it takes them 256 at a time)."""
    frames = [scenes.random_frame(seed, W=16, H=16, depth_range=(1.0, 10.0), fx=4.0, translation_scale=0.3)
              for seed in (11, 12)]
    frames.append(scenes.random_frame(13, W=32, H=32, depth_range=(1.0, 10.0), fx=8.0, translation_scale=0.3))
    _, st, coords, arrays, o = run_both(frames[:1], 0.01, 0.04, 1 << 16, mode=mode)
    assert st["pool_used"] > 800                 # one tile: its filings pass 256 keys at a time
    assert_parity(st, coords, arrays, o)
    _, st, coords, arrays, o = run_both(frames, 0.01, 0.04, 1 << 16, mode=mode, batch=3)
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
def test_long_walks_parity(mode):
    """Bands many voxels deep, so walks run through several of allocate's
    31-cell chunks: every chunk after the first is filed separately and
    starts from a walk set up again and replayed to where the last one
    stopped.  Block set, weights and counts must still match exactly."""
    frames = [scenes.random_frame(90 + j, W=37, H=23, invalid_frac=0.1, translation_scale=0.5)
              for j in range(3)]
    for vs, tr in ((0.01, 0.2), (0.005, 0.31)):
        _, st, coords, arrays, o = run_both(frames, vs, tr, 1 << 18, mode=mode)
        assert st["walk_guard"] == 0
        assert_parity(st, coords, arrays, o)


def _frame_like(base, depth, t=None):
    H, W = depth.shape
    rgb = np.resize(base.rgb, (H, W, 3)).astype(np.uint8) if H * W else np.zeros((H, W, 3), np.uint8)
    return scenes.Frame(np.ascontiguousarray(depth, np.float32), rgb, base.fx, base.fy, base.cx, base.cy,
                        base.R, base.t if t is None else np.asarray(t, np.float32))


@pytest.mark.parametrize("mode", MODES)
def test_edge_inputs(mode):
    base = scenes.random_frame(21, W=9, H=6)
    vs, tr = 0.01, 0.04
    nan = np.full((6, 9), np.nan)
    nan[0, :4] = [np.inf, -np.inf, -1.0, 0.0]
    near = np.full((6, 9), 0.03)
    cases = {
        "empty": np.zeros((0, 0)),
        "zeros": np.zeros((6, 9)),
        "nonfinite": nan,
        "near": near,
        "mixed": np.where(np.arange(54).reshape(6, 9) % 3 == 0, base.depth, near),
    }
    for name, d in cases.items():
        say(f"  edge case {name}")
        _, st, coords, arrays, o = run_both([_frame_like(base, d)], vs, tr, 1024, mode=mode)
        assert_parity(st, coords, arrays, o)
    say("  edge case out of range")
    fr = _frame_like(base, base.depth, t=[1e5, 0.0, 0.0])
    _, st, coords, arrays, o = run_both([fr], vs, tr, 1024, mode=mode)
    assert st["out_of_range"] == 54 and st["pool_used"] == 0
    assert_parity(st, coords, arrays, o)
    say("  edge case far but in range")
    fr = _frame_like(base, base.depth, t=[80000.0, -80000.0, 80000.0])
    _, st, coords, arrays, o = run_both([fr], vs, tr, 1024, mode=mode)
    assert st["points_valid"] == 54
    assert_parity(st, coords, arrays, o)


@pytest.mark.parametrize("mode", MODES)
def test_band_ends_and_far_poses(mode):
    """Cells whose centres lie exactly on the band's ends, and cameras far
    from the origin (a wide margin around the ends): the walk's band
    decisions, taken on a stepped sdf away from the ends, must be the exact
    test's everywhere."""
    vs, tr = 2.0 ** -7, 2.0 ** -5
    W, H = 48, 40
    rng = np.random.default_rng([11, 3])
    k = rng.integers(40, 200, size=(H, W))
    # grid-aligned cameras: a centre's camera depth is a world coordinate
    # plus a lattice offset, (k + 1/2) vs exactly, and so is every sdf, many
    # of them exactly +-trunc
    depth = ((k + 0.5) * vs + tr).astype(np.float32)
    rgb = rng.integers(0, 256, size=(H, W, 3), dtype=np.uint8)
    cyclic = np.array([[0, 0, 1], [1, 0, 0], [0, 1, 0]], np.float32)   # camera z along world x
    for name, R, t in (("identity", np.eye(3, dtype=np.float32), np.zeros(3, np.float32)),
                       ("axis permutation", cyclic, np.array([-3.0, 0.5, 1.25], np.float32))):
        fr = scenes.Frame(depth, rgb, 40.0, 40.0, 23.5, 19.5, R, t)
        say(f"  grid-aligned camera ({name}), depths on the voxel lattice")
        _, st, coords, arrays, o = run_both([fr], vs, tr, 1 << 16, mode=mode)
        assert st["points_valid"] == W * H
        assert_parity(st, coords, arrays, o)
    for seed, dist in ((31, 40.0), (32, 300.0)):
        base = scenes.random_frame(seed, W=33, H=21)
        fr = scenes.Frame(base.depth, base.rgb, base.fx, base.fy, base.cx, base.cy, base.R,
                          np.asarray(base.t, np.float32) + np.float32(dist))
        say(f"  camera {dist:g} m out on each axis")
        _, st, coords, arrays, o = run_both([fr], 0.01, 0.04, 1 << 16, mode=mode)
        assert_parity(st, coords, arrays, o)


# ---------------------------------------------------------------------------
# loss accounting, protocol and API behaviour
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
def test_pool_exhaustion_is_counted_exactly(mode):
    wl = scenes.workload("spherewall320x240")
    frames = list(wl.frames(0, 3))
    n = parity.oracle_integrate(frames, wl.voxel_size, wl.trunc, 1 << 20).block_count()
    cap = n - 100
    _, st, coords, arrays, o = run_both(frames, wl.voxel_size, wl.trunc, cap, table=scenes.next_pow2(2 * n),
                                        mode=mode)
    assert st["pool_used"] == cap and st["pool_overflow"] == 100
    assert st["table_full"] == 0
    w = arrays["weight"].astype(np.float64)
    assert int(w.sum()) + st["update_misses"] == st["voxel_updates"] == o.totals()["voxel_updates"]
    assert np.all(w.max(1) > 0)                      # every block that got an index got contributions
    assert len(np.unique(coords, axis=0)) == cap
    _survivors_exact(frames, wl.voxel_size, wl.trunc, st, coords, arrays)


def _survivors_exact(frames, vs, tr, st, coords, arrays):
    """A block's contributions do not depend on which other keys an exhausted
    pool or a full table refused: every block the GPU kept equals that block
    of an oracle run with unlimited capacity, and the refused blocks' weight
    is exactly the counted misses."""
    full = parity.oracle_integrate(frames, vs, tr, 1 << 24)
    keep = {tuple(c) for c in coords.tolist()}
    allc = {tuple(c) for c in full.block_coords().tolist()}
    assert keep <= allc
    lost = sorted(allc - keep)
    w_lost = float(full.block_sums(np.array(lost, np.int32).reshape(-1, 3))["weight"].sum()) if lost else 0.0
    assert st["update_misses"] == w_lost
    f = parity.compare_blocks(coords, arrays, _OracleSubset(full, keep))
    assert f == [], f


@pytest.mark.parametrize("mode", MODES)
def test_full_table_terminates_and_counts(mode):
    # 2-entry table: the probe must stop after trying both slots, never hang
    base = scenes.random_frame(5, W=16, H=16)
    _, st, coords, arrays, o = run_both([base], 0.01, 0.04, 1, table=2, mode=mode)
    assert st["pool_used"] == 1 and st["pool_overflow"] == 1
    assert st["table_full"] > 0
    assert int(arrays["weight"].astype(np.float64).sum()) + st["update_misses"] == st["voxel_updates"]
    assert st["voxel_updates"] == o.totals()["voxel_updates"]
    _survivors_exact([base], 0.01, 0.04, st, coords, arrays)


@pytest.mark.parametrize("mode", MODES)
def test_second_allocate_inserts_nothing_and_reset(mode):
    import torch
    from hash_table_amd import tsdf
    wl = scenes.workload("spherewall320x240")
    f0 = tsdf.DeviceFrame(wl.frame(0))
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, update_mode=mode)
    vol.allocate(f0)
    st1 = vol.stats()
    vol.allocate(f0)
    st = vol.stats()
    assert st["pool_used"] == st1["pool_used"] > 0 and st["pool_overflow"] == 0
    assert st["voxel_updates"] == 2 * st1["voxel_updates"]     # every allocate counts its frame
    vol.update(f0)
    c1, a1 = parity.sort_blocks(*vol.export())
    assert float(a1["weight"].sum()) == st1["voxel_updates"]      # but the frame was added once
    vol.reset()
    assert vol.stats()["pool_used"] == 0
    vol.integrate(f0)
    torch.cuda.synchronize()
    c2, a2 = parity.sort_blocks(*vol.export())
    assert np.array_equal(c1, c2) and np.array_equal(a1["weight"], a2["weight"])


def test_owner_update_must_follow_its_allocate():
    from hash_table_amd import tsdf
    wl = scenes.workload("spherewall320x240")
    f0, f1 = tsdf.DeviceFrame(wl.frame(0)), tsdf.DeviceFrame(wl.frame(1))
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, update_mode="owner")
    with pytest.raises(tsdf.TsdfError):
        vol.update(f0)                                # no allocate yet
    vol.allocate(f0)
    with pytest.raises(tsdf.TsdfError):
        vol.update(f1)                                # a different frame
    vol.update(f0)
    with pytest.raises(tsdf.TsdfError):
        vol.update(f0)                                # already added
    assert vol.stats()["pool_used"] > 0


def test_unwritten_blocks_of_a_dropped_allocate():
    # frame 1's allocate is dropped (another allocate follows it): its new
    # blocks hold pool indices but no sums; the next calls must still add to
    # them correctly (they are still zero), and the result is frames 0, 3, 1
    # and 2 integrated once each; then the same after a reset
    from hash_table_amd import tsdf
    wl = scenes.workload("spherewall320x240")
    host = [wl.frame(i) for i in range(4)]
    f = [tsdf.DeviceFrame(h) for h in host]
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, update_mode="owner")
    for rep in range(2):
        vol.integrate(f[0])
        vol.allocate(f[1])                            # dropped by the next allocate
        vol.allocate(f[3])
        vol.update(f[3])
        vol.integrate_batch([f[1], f[2]])
        coords, arrays = vol.export()
        o = parity.oracle_integrate([host[0], host[3], host[1], host[2]], wl.voxel_size, wl.trunc,
                                    wl.pool_capacity)
        # (the dropped allocate counted its points: compare blocks and sums)
        bad = parity.compare_blocks(coords, arrays, o)
        assert bad == [], bad
        vol.reset()


def test_repeat_runs_identical_blocks_and_weights():
    wl = scenes.workload("cube640x480")
    f = wl.frame(0)
    r1 = parity.gpu_integrate([f], wl.voxel_size, wl.trunc, wl.pool_capacity)
    r2 = parity.gpu_integrate([f], wl.voxel_size, wl.trunc, wl.pool_capacity)
    c1, a1 = parity.sort_blocks(r1[2], r1[3])
    c2, a2 = parity.sort_blocks(r2[2], r2[3])
    assert np.array_equal(c1, c2) and np.array_equal(a1["weight"], a2["weight"])
    for n in parity.CHANNELS:                        # sums may differ only by summation order
        m = a1["weight"] > 0
        assert np.abs(a1[n][m] / a1["weight"][m] - a2[n][m] / a2["weight"][m]).max() <= parity.MEAN_TOL


def test_export_too_small_and_invalid_frames():
    import torch
    from hash_table_amd import tsdf
    wl = scenes.workload("plane64x48")
    f = tsdf.DeviceFrame(wl.frame(0))
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity)
    vol.integrate(f)
    c = torch.empty((10, 3), dtype=torch.int32, device="cuda")
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_export_blocks(vol.handle, c.data_ptr(), 0, 0, 0, 0, 0, 10)
    assert e.value.status == tsdf.TSDF_ESMALL
    bad = tsdf.DeviceFrame(wl.frame(0))
    bad.desc.fx = 0.0
    with pytest.raises(tsdf.TsdfError):
        vol.integrate(bad)
    bad = tsdf.DeviceFrame(wl.frame(0))
    bad.desc.R[4] = float("nan")
    with pytest.raises(tsdf.TsdfError):
        vol.update(bad)
    bad = tsdf.DeviceFrame(wl.frame(0))
    bad.desc.fx = 1e-3                               # a walk longer than TSDF_MAX_WALK cells
    with pytest.raises(tsdf.TsdfError):
        vol.allocate(bad)
    bad = tsdf.DeviceFrame(wl.frame(0))
    bad.desc.rgb = None
    with pytest.raises(tsdf.TsdfError):
        vol.update(bad)
    vol.allocate(bad)                                # allocate does not need colour
    assert vol.stats()["pool_used"] == 234
    bad = tsdf.DeviceFrame(wl.frame(0))
    bad.desc.R[0] = 2.0                              # not a rotation
    with pytest.raises(tsdf.TsdfError):
        vol.allocate(bad)
    # wider than TSDF_MAX_FRAME_SIDE: refused before any launch (the buffers
    # are sized for the frame anyway, all depths 0, so nothing can read past them)
    wide = scenes.Frame(np.zeros((1, tsdf.TSDF_MAX_FRAME_SIDE + 1), np.float32),
                        np.zeros((1, tsdf.TSDF_MAX_FRAME_SIDE + 1, 3), np.uint8),
                        1000.0, 1000.0, 0.0, 0.0, np.eye(3, dtype=np.float32), np.zeros(3, np.float32))
    with pytest.raises(tsdf.TsdfError) as e:
        vol.allocate(tsdf.DeviceFrame(wide))
    assert e.value.status == tsdf.TSDF_EINVAL


@pytest.mark.parametrize("mode", MODES)
def test_kernel_timing(mode):
    import torch
    from hash_table_amd import tsdf
    wl = scenes.workload("spherewall320x240")
    frames = [tsdf.DeviceFrame(wl.frame(i)) for i in range(3)]
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, update_mode=mode)
    with pytest.raises(tsdf.TsdfError):
        vol.kernel_times()                            # timing is off
    vol.set_kernel_timing(True)
    vol.integrate_batch(frames)
    vol.integrate(frames[0])
    kt = vol.kernel_times()
    say(f"  kernel times ({mode}): {kt}")
    expect = {"k_allocate", "k_place_items", "k_place_segments", "k_update_owner", "k_update_rescan"} \
        if mode == "owner" else {"k_allocate", "k_update_rays"}
    assert set(kt) == expect
    for v in kt.values():
        assert v["launches"] == 2 and v["total_ms"] > 0.0
    assert vol.kernel_times() == {}                   # read sums are cleared
    vol.set_kernel_timing(False)
    torch.cuda.synchronize()
