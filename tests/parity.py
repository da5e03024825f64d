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


def oracle_integrate(frames: Iterable, voxel_size, trunc, pool_capacity, reproject=False) -> oracle.Oracle:
    o = oracle.Oracle(voxel_size, trunc, pool_capacity, reproject=reproject)
    for f in frames:
        o.integrate(f)
    return o


def compare_blocks(coords, arrays, o: oracle.Oracle, sample: Optional[np.ndarray] = None,
                   errors: Optional[dict] = None) -> List[str]:
    """Compare an exported GPU volume with the oracle.  `sample` restricts the
    per-voxel comparison to those blocks (the block SET is always compared in
    full).  `errors`, if given, receives the largest mean difference per
    channel."""
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
            if errors is not None:
                errors[n] = float(err)
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


# ---------------------------------------------------------------------------
# long sequences: the oracle on disjoint frame ranges in worker processes
# ---------------------------------------------------------------------------
def _pack(coords: np.ndarray) -> np.ndarray:
    c = coords.astype(np.int64) + (1 << 20)
    return c[:, 0] | (c[:, 1] << 21) | (c[:, 2] << 42)


def _oracle_range(args):
    """Worker: render frames [a, b) of a named workload, integrate them with
    the (unchanged, single-threaded) oracle into a fresh volume, and return
    the frames, the block coordinates, their sums and the totals."""
    name, a, b = args
    from hash_table_amd import scenes
    wl = scenes.workload(name)
    frames = [wl.frame(i) for i in range(a, b)]
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity)
    for f in frames:
        o.integrate(f)
    coords = o.block_coords()
    return a, frames, coords, o.block_sums(coords), o.totals()


class SummedOracle:
    """The oracle's result for a whole frame sequence, assembled from oracle
    runs over disjoint frame ranges: the union of their block sets, and per
    voxel the sum of their sums.  The contributions of the frames are the same
    terms the single run adds (sums commute; the oracle's own pins check that
    the result does not depend on frame order), so this equals one run over
    all frames up to float64 rounding of the additions, with exact weights.
    Only valid when no pool capacity is reached (every key gets a block)."""

    def __init__(self, parts, capacity):
        keys = np.unique(np.concatenate([_pack(c) for _, c, _, _ in parts]))
        n = len(keys)
        self._coords = np.empty((n, 3), np.int32)
        self._sums = {k: np.zeros((n, 512), np.float64) for k in ("tsdf", "weight", "r", "g", "b")}
        self._tot = {"blocks": n, "pool_overflow": 0, "update_misses": 0, "points_valid": 0, "near_skipped": 0,
                     "out_of_range": 0, "voxel_updates": 0, "frames": 0}
        for _, c, sums, tot in parts:
            idx = np.searchsorted(keys, _pack(c))
            self._coords[idx] = c
            for k, v in sums.items():
                self._sums[k][idx] += v
            for k in ("points_valid", "near_skipped", "out_of_range", "voxel_updates", "frames", "update_misses"):
                self._tot[k] += tot[k]
            assert tot["pool_overflow"] == 0
        assert n <= capacity, "a capacity-bound sequence cannot be split"
        order = np.lexsort((self._coords[:, 2], self._coords[:, 1], self._coords[:, 0]))
        self._coords = self._coords[order]
        self._sums = {k: v[order] for k, v in self._sums.items()}
        self._row = {k: i for i, k in enumerate(_pack(self._coords).tolist())}

    def totals(self):
        return dict(self._tot)

    def block_count(self):
        return len(self._coords)

    def block_coords(self):
        return self._coords

    def block_sums(self, coords):
        rows = [self._row.get(k, -1) for k in _pack(np.asarray(coords).reshape(-1, 3)).tolist()]
        out = {}
        for k, v in self._sums.items():
            a = v[np.maximum(rows, 0)] if rows else np.empty((0, 512))
            a[np.asarray(rows) < 0] = np.nan
            out[k] = a
        return out


def oracle_ranges(name: str, n_frames: int, workers: int = 8):
    """Run the oracle over frames [0, n_frames) of workload `name` split into
    `workers` contiguous ranges, one worker process each (spawned: the
    workers load no GPU library).  Returns (frames in order, SummedOracle)."""
    import multiprocessing as mp
    from hash_table_amd import scenes
    wl = scenes.workload(name)
    b = [round(i * n_frames / workers) for i in range(workers + 1)]
    jobs = [(name, b[i], b[i + 1]) for i in range(workers) if b[i + 1] > b[i]]
    ctx = mp.get_context("spawn")
    parts = []
    frames = {}
    with ctx.Pool(len(jobs)) as pool:
        for a, fr, coords, sums, tot in pool.imap_unordered(_oracle_range, jobs):
            say(f"    oracle frames {a}..{a + len(fr) - 1}: {len(coords)} blocks")
            for i, f in enumerate(fr):
                frames[a + i] = f
            parts.append((a, coords, sums, tot))
    return [frames[i] for i in range(n_frames)], SummedOracle(parts, wl.pool_capacity)


# ---------------------------------------------------------------------------
# the hash table itself: linear probing leaves a layout that does not depend
# on the order of the insertions
# ---------------------------------------------------------------------------
_M1, _M2 = np.uint64(0xFF51AFD7ED558CCD), np.uint64(0xC4CEB9FE1A85EC53)


def fmix64(k: np.ndarray) -> np.ndarray:
    """The 64-bit finaliser of MurmurHash3 (the table's home-slot hash)."""
    k = k.astype(np.uint64).copy()
    with np.errstate(over="ignore"):
        k ^= k >> np.uint64(33)
        k *= _M1
        k ^= k >> np.uint64(33)
        k *= _M2
        k ^= k >> np.uint64(33)
    return k


def table_layout_failures(table_words: np.ndarray, coords: np.ndarray, capacity: int) -> List[str]:
    """Check an exported hash table (2 x uint64 per entry: key, index word)
    against the keys it must hold.  Linear probing from the home slots fills
    a set of slots that is the same whatever order the keys arrive in, and
    the total displacement (slots past the home slot, summed over keys) is the
    same too; every key sits at or after its home slot with no empty slot in
    between; pool indices are distinct and below the capacity."""
    f = []
    T = table_words.shape[0]
    mask = np.uint64(T - 1)
    tk = table_words[:, 0].astype(np.uint64)
    occupied = tk != np.uint64(0xFFFFFFFFFFFFFFFF)
    keys = _pack(coords).astype(np.uint64)
    home = (fmix64(keys) & mask).astype(np.int64)
    slot_of = {int(k): i for i, k in enumerate(tk[occupied].tolist())}
    occ_slots = np.nonzero(occupied)[0]
    if occupied.sum() != len(keys):
        f.append(f"table holds {int(occupied.sum())} keys, expected {len(keys)}")
        return f
    try:
        pos = np.array([occ_slots[slot_of[int(k)]] for k in keys.tolist()], np.int64)
    except KeyError as e:
        f.append(f"key {e} missing from the table")
        return f
    # the order-independent layout: insert in sorted-key order on the host
    want = np.zeros(T, bool)
    disp_want = 0
    for h in np.sort(home):
        p = int(h)
        while want[p]:
            p = (p + 1) & (T - 1)
        want[p] = True
        disp_want += (p - int(h)) & (T - 1)
    if not np.array_equal(want, occupied):
        f.append("occupied slots differ from linear probing's order-independent layout")
    disp = (pos - home) & (T - 1)
    if int(disp.sum()) != disp_want:
        f.append(f"total displacement {int(disp.sum())} != {disp_want}")
    for p, h in zip(pos.tolist(), home.tolist()):       # no hole between home and position
        q = h
        while q != p:
            if not occupied[q]:
                f.append(f"empty slot {q} between a key's home {h} and its slot {p}")
                return f
            q = (q + 1) & (T - 1)
    idx = (table_words[occupied, 1].astype(np.uint64) & np.uint64(0xFFFFFFFF)).astype(np.int64)
    if len(np.unique(idx)) != len(idx) or (len(idx) and idx.max() >= capacity):
        f.append("pool indices repeat or exceed the capacity")
    return f
