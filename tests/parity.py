"""Helpers that run the HIP library and the oracle on the same seeded frames
and compare them element by element.

The bar: block set, block count and per-voxel weights bit-exact (weights are
integer-valued floats); mean TSDF and mean colour (sum / weight) within 1e-4
absolute, because float atomic summation order differs; every loss counter
equal to the oracle's (zero unless the case exhausts the pool on purpose).
"""
from __future__ import annotations

import sys
from typing import Dict, Iterable, List, Optional

import numpy as np

import oracle

MEAN_TOL = 1e-4
CHANNELS = ("tsdf", "r", "g", "b")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sort_blocks(coords: np.ndarray, arrays: Dict[str, np.ndarray]):
    order = np.lexsort((coords[:, 2], coords[:, 1], coords[:, 0]))
    return coords[order], {k: v[order] for k, v in arrays.items()}


def gpu_integrate(frames: Iterable, voxel_size, trunc, pool_capacity, table_entries=0, split=False,
                  per_frame_stats=False, mode="owner", batch=1, max_batch_pixels=0, occlusion="ray"):
    """Integrate on the GPU (one frame per call, or `batch` frames per
    tsdf_integrate_batch call); returns (volume, stats, coords, arrays,
    per-call stats)."""
    import torch
    from hash_table_amd import tsdf
    frames = list(frames)
    vol = tsdf.Volume(voxel_size, trunc, pool_capacity, table_entries, update_mode=mode,
                      max_batch_pixels=max_batch_pixels, occlusion=occlusion)
    history = []
    if batch > 1:
        for i in range(0, len(frames), batch):
            dfs = [tsdf.DeviceFrame(f) for f in frames[i:i + batch]]
            vol.integrate_batch(dfs)
            if per_frame_stats:
                history.append(vol.stats())
    for f in (frames if batch <= 1 else []):
        df = tsdf.DeviceFrame(f)
        if split:
            vol.allocate(df)
            vol.update(df)
        else:
            vol.integrate(df)
        if per_frame_stats:
            history.append(vol.stats())
    torch.cuda.synchronize()
    st = vol.stats()
    coords, arrays = vol.export()
    return vol, st, coords, arrays, history


def oracle_integrate(frames: Iterable, voxel_size, trunc, pool_capacity, watch=None,
                     reproject=False) -> oracle.Oracle:
    o = oracle.Oracle(voxel_size, trunc, pool_capacity, watch=watch, reproject=reproject)
    for f in frames:
        o.integrate(f)
    return o


def compare_blocks(coords, arrays, o: oracle.Oracle, sample: Optional[np.ndarray] = None) -> List[str]:
    """Compare an exported GPU volume with the oracle.  `sample` restricts the
    per-voxel comparison to those blocks (the block SET is always compared in
    full)."""
    f = []
    gc, ga = sort_blocks(coords, arrays)
    if len(np.unique(gc, axis=0)) != len(gc):
        f.append("duplicate block coordinates in the export")
    oc = o.block_coords()
    if gc.shape != oc.shape or not np.array_equal(gc, oc):
        gs = {tuple(x) for x in gc.tolist()}
        os_ = {tuple(x) for x in oc.tolist()}
        f.append(f"block sets differ: gpu {len(gs)} oracle {len(os_)}, gpu-only {sorted(gs - os_)[:3]}, "
                 f"oracle-only {sorted(os_ - gs)[:3]}")
        return f
    if sample is not None:
        keep = np.zeros(len(gc), bool)
        sset = {tuple(x) for x in np.asarray(sample).tolist()}
        for i, c in enumerate(gc.tolist()):
            keep[i] = tuple(c) in sset
        gc = gc[keep]
        ga = {k: v[keep] for k, v in ga.items()}
    s = o.block_sums(gc)
    gw = ga["weight"].astype(np.float64)
    if np.isnan(s["weight"]).any():
        f.append("oracle has no sums for some compared blocks")
        return f
    if not np.array_equal(gw, s["weight"]):
        bad = np.argwhere(gw != s["weight"])
        i, j = bad[0]
        f.append(f"weights differ at {len(bad)} voxels, e.g. block {gc[i].tolist()} voxel {j}: "
                 f"gpu {gw[i, j]} oracle {s['weight'][i, j]}")
        return f
    m = gw > 0
    for n in CHANNELS:
        g = ga[n].astype(np.float64)
        if np.any(g[~m] != 0.0):
            f.append(f"{n}: nonzero sum at a voxel with zero weight")
        if m.any():
            err = np.abs(g[m] / gw[m] - s[n][m] / gw[m]).max()
            if not err <= MEAN_TOL:
                f.append(f"mean {n} differs by {err:.3g} (> {MEAN_TOL})")
    return f


def compare_stats(st: dict, o: oracle.Oracle, expect_loss: bool = False) -> List[str]:
    f = []
    tot = o.totals()
    for g, k in (("points_valid", "points_valid"), ("voxel_updates", "voxel_updates"),
                 ("near_skipped", "near_skipped"), ("out_of_range", "out_of_range")):
        if st[g] != tot[k]:
            f.append(f"{g}: gpu {st[g]} oracle {tot[k]}")
    if st["pool_used"] != tot["blocks"]:
        f.append(f"pool_used: gpu {st['pool_used']} oracle {tot['blocks']}")
    if st["pool_overflow"] != tot["pool_overflow"]:
        f.append(f"pool_overflow: gpu {st['pool_overflow']} oracle {tot['pool_overflow']}")
    if st["walk_guard"] != 0:
        f.append(f"walk_guard {st['walk_guard']}")
    if not expect_loss:
        for k in ("table_full", "update_misses", "pool_overflow"):
            if st[k] != 0:
                f.append(f"{k} = {st[k]} (expected no loss)")
    return f
