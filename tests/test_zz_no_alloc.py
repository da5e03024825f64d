"""tsdf_integrate_batch_noalloc (the entry point for callers that cannot
allocate) against tsdf_integrate_batch, through the C ABI (needs an MI355X).

Two volumes of one configuration integrate the same frames, one with each
entry point, in two calls in a row (the second smaller): after each call the
statistics agree and the exported volumes agree block by block (block set,
weights bit-exact, means within 1e-4).  One volume mixing both entry points
(whose fresh-block bookkeeping the no-allocation call must hand back) matches
the oracle.  The limits are refused without launching anything.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from hash_table_amd import scenes
from tests import parity
from tests.parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build()


def _same_volume(a_stats, a, b_stats, b, label):
    # (fallback_blocks is not compared: when run records overflow, which
    # blocks are rescanned depends on the order of the atomics; both are exact)
    for k in ("pool_used", "pool_overflow", "table_full", "update_misses", "points_valid", "voxel_updates",
              "near_skipped", "out_of_range", "walk_guard"):
        assert a_stats[k] == b_stats[k], f"{label}: {k} {a_stats[k]} != {b_stats[k]}"
    (ca, xa), (cb, xb) = (parity.sort_blocks(*a), parity.sort_blocks(*b))
    assert np.array_equal(ca, cb), f"{label}: block sets differ"
    assert np.array_equal(xa["weight"], xb["weight"]), f"{label}: weights differ"
    w = xa["weight"].astype(np.float64)
    m = w > 0
    for n in parity.CHANNELS:
        err = np.abs(xa[n].astype(np.float64)[m] / w[m] - xb[n].astype(np.float64)[m] / w[m]).max()
        assert err <= parity.MEAN_TOL, f"{label}: mean {n} differs by {err:.3g}"


@pytest.mark.parametrize("mode", ["owner", "rays"])
def test_noalloc_matches_integrate_batch(mode):
    import torch
    from hash_table_amd import tsdf
    wl = scenes.workload("spherewall320x240")
    frames = [tsdf.DeviceFrame(wl.frame(i)) for i in range(6)]
    sh = torch.cuda.current_stream().cuda_stream
    vols = [tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, update_mode=mode, max_batch_pixels=5 * 320 * 240)
            for _ in range(2)]
    for calls, label in (([0, 1, 2, 3, 4], "call 1 (5 frames)"), ([5], "call 2 (1 frame)")):
        descs = [frames[i].desc for i in calls]
        say(f"  {mode}: {label}")
        tsdf.tsdf_integrate_batch(vols[0].handle, descs, sh)
        tsdf.tsdf_integrate_batch_noalloc(vols[1].handle, descs, sh)
        torch.cuda.synchronize()
        _same_volume(vols[0].stats(), vols[0].export(), vols[1].stats(), vols[1].export(), f"{mode} {label}")


def test_noalloc_mixed_with_other_entry_points():
    """normal, no-allocation, normal (split allocate / update), no-allocation:
    the volume equals the oracle's over all frames, so every call wrote its
    blocks' first sums exactly once and added to older ones."""
    import torch
    from hash_table_amd import tsdf
    wl = scenes.workload("spherewall320x240")
    host = [wl.frame(i) for i in range(8)]
    frames = [tsdf.DeviceFrame(f) for f in host]
    sh = torch.cuda.current_stream().cuda_stream
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, max_batch_pixels=3 * 320 * 240)
    tsdf.tsdf_integrate_batch(vol.handle, [f.desc for f in frames[0:2]], sh)
    tsdf.tsdf_integrate_batch_noalloc(vol.handle, [f.desc for f in frames[2:5]], sh)
    tsdf.tsdf_allocate_batch(vol.handle, [f.desc for f in frames[5:7]], sh)
    tsdf.tsdf_update_batch(vol.handle, [f.desc for f in frames[5:7]], sh)
    tsdf.tsdf_allocate_batch(vol.handle, [frames[7].desc], sh)       # dropped: no update follows
    tsdf.tsdf_integrate_batch_noalloc(vol.handle, [frames[7].desc], sh)
    torch.cuda.synchronize()
    st = vol.stats()
    coords, arrays = vol.export()
    o = parity.oracle_integrate(host, wl.voxel_size, wl.trunc, wl.pool_capacity)
    f = parity.compare_stats({**st, "points_valid": st["points_valid"] - o.frame_stats[7]["points_valid"],
                              "voxel_updates": st["voxel_updates"] - o.frame_stats[7]["voxel_updates"]}, o)
    f += parity.compare_blocks(coords, arrays, o)
    assert f == [], f


@pytest.mark.parametrize("mode", ["owner", "rays"])
def test_noalloc_call_of_many_frames(mode):
    """A 40-frame call (frames 32.. travel in the device frame table, written
    by the call's own kernels) matches tsdf_integrate_batch."""
    import torch
    from hash_table_amd import tsdf
    host = [scenes.random_frame(200 + i, W=37, H=23, translation_scale=0.5) for i in range(40)]
    frames = [tsdf.DeviceFrame(f) for f in host]
    sh = torch.cuda.current_stream().cuda_stream
    vols = [tsdf.Volume(0.013, 0.052, 1 << 18, update_mode=mode, max_batch_pixels=40 * 37 * 23) for _ in range(2)]
    descs = [f.desc for f in frames]
    tsdf.tsdf_integrate_batch(vols[0].handle, descs, sh)
    tsdf.tsdf_integrate_batch_noalloc(vols[1].handle, descs, sh)
    torch.cuda.synchronize()
    _same_volume(vols[0].stats(), vols[0].export(), vols[1].stats(), vols[1].export(), f"{mode} 40 frames")
    o = parity.oracle_integrate(host, 0.013, 0.052, 1 << 18)
    f = parity.compare_stats(vols[1].stats(), o) + parity.compare_blocks(*vols[1].export(), o)
    assert f == [], f


def test_noalloc_limits():
    import torch
    from hash_table_amd import tsdf
    sh = torch.cuda.current_stream().cuda_stream
    wl = scenes.workload("spherewall320x240")
    f = tsdf.DeviceFrame(wl.frame(0))
    vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity)
    with pytest.raises(tsdf.TsdfError) as e:                      # more frames than a call takes
        tsdf.tsdf_integrate_batch_noalloc(vol.handle, [f.desc] * (tsdf.TSDF_MAX_BATCH + 1), sh)
    assert e.value.status == tsdf.TSDF_EINVAL
    # a call whose work lists exceed the fixed scratch: a 2^21-entry table
    # (120 MB of per-slot lists) is refused, nothing enqueued
    big = tsdf.Volume(0.005, 0.02, 1 << 20)
    with pytest.raises(tsdf.TsdfError) as e:
        tsdf.tsdf_integrate_batch_noalloc(big.handle, [f.desc], sh)
    assert e.value.status == tsdf.TSDF_ELIMIT
    torch.cuda.synchronize()
    assert vol.stats()["points_valid"] == 0 and big.stats()["points_valid"] == 0
    # the limit is the documented size: 32 frames of this volume fit or not by tsdf_scratch_bytes
    cfg = tsdf.tsdf_config(wl.voxel_size, wl.trunc, wl.pool_capacity, 0, tsdf.TSDF_UPDATE_OWNER, 32 * 320 * 240)
    need = tsdf.tsdf_scratch_bytes(cfg)
    if need <= tsdf.TSDF_NOALLOC_SCRATCH_BYTES:
        tsdf.tsdf_integrate_batch_noalloc(vol.handle, [f.desc] * 32, sh)
    else:
        with pytest.raises(tsdf.TsdfError) as e:
            tsdf.tsdf_integrate_batch_noalloc(vol.handle, [f.desc] * 32, sh)
        assert e.value.status == tsdf.TSDF_ELIMIT
    torch.cuda.synchronize()
