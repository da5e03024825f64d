"""Write the stored expected counts under tests/golden/ by running ONLY the
oracle on the seeded synthetic workloads.

    python tests/golden/make_golden.py [workload ...]
    python tests/golden/make_golden.py sweep      # the benchmark's sweep cells
    python tests/golden/make_golden.py calls [workload ...]   # per-call counts of the benchmark's calls

For each workload it writes <name>_counts.json: per frame the SHA-256 of the
generated inputs and the oracle's exact integer counts (valid points, voxel
updates V, distinct voxels U, blocks touched B_t, new blocks B_n, cells
visited) plus the running block count.  The load-factor tests pick their
pool sizes and frame prefixes from the running block count, and the
benchmark takes its algorithmic byte counts (depth/colour per pixel, one
16-byte table entry per touched block, one more per new block, five floats
read and written per touched voxel) from these numbers.  calls.json holds,
for each way the benchmark splits a workload into calls, the counts of each
call: the compulsory traffic of a batched call depends on the distinct
blocks and voxels of the call, not of each frame.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from hash_table_amd import scenes  # noqa: E402


def frame_sha(f) -> str:
    return scenes.frame_digest([f])


def make_counts(name: str, n_frames=None) -> dict:
    wl = scenes.workload(name)
    n = wl.n_frames if n_frames is None else min(n_frames, wl.n_frames)
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity, track_touched=True)
    frames = []
    t_oracle = 0.0
    for i in range(n):
        f = wl.frame(i)
        t0 = time.perf_counter()
        st = o.integrate(f)
        t_oracle += time.perf_counter() - t0
        st["blocks_total"] = o.block_count()
        st["sha256"] = frame_sha(f)
        frames.append(st)
        print(f"{name} frame {i}: V={st['voxel_updates']} U={st['voxels_touched']} "
              f"B_t={st['blocks_touched']} blocks={st['blocks_total']}", flush=True)
    return {
        "workload": name,
        "voxel_size": wl.voxel_size, "trunc": wl.trunc,
        "pool_capacity": wl.pool_capacity, "table_entries": wl.table_entries,
        "width": wl.width, "height": wl.height, "n_frames": n,
        "totals": o.totals(),
        "oracle_seconds_here": round(t_oracle, 2),
        "frames": frames,
        "written_by": "tests/golden/make_golden.py (oracle only)",
    }


SWEEP_FRAMES = 16     # frames of each sweep cell (one batched call)
CALLS_PATH = os.path.join(HERE, "calls.json")


def call_counts(name: str, calls) -> list:
    """The oracle's counts of each call of a split (contiguous frame ranges,
    integrated in order into one volume, a call boundary between ranges):
    frames, pixels, valid points, voxel updates, distinct blocks touched,
    blocks created, distinct voxels touched in blocks the call created and in
    older ones."""
    wl = scenes.workload(name)
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity, track_touched=True)
    out = []
    for j, (a, b) in enumerate(calls):
        if j:
            o.begin_call()
        pixels = points = updates = 0
        for i in range(a, b):
            st = o.integrate(wl.frame(i))
            pixels += st["pixels"]
            points += st["points_valid"]
            updates += st["voxel_updates"]
        c = o.call_stats()
        c.update({"first": a, "end": b, "pixels": pixels, "points_valid": points, "voxel_updates": updates})
        out.append(c)
        print(f"{name} call {a}..{b - 1}: {c}", flush=True)
    return out


def bench_splits():
    """Every (workload, split name, calls) the benchmark times."""
    out = [(n, f"{len(c)}x{c[0][1] - c[0][0]}", c) for n, c in scenes.BENCH_CALLS.items()]
    with open(os.path.join(HERE, "room640x480_counts.json")) as fh:
        totals = [f["blocks_total"] for f in json.load(fh)["frames"]]
    for lf in scenes.LOAD_FACTORS:
        _, n, _ = scenes.load_factor_cell(totals, lf)
        out.append(("room640x480", f"prefix{n}", [(0, n)]))
    for _, W, H, fx in scenes.SWEEP_CELLS:
        if (W, H) != (640, 480):
            out.append((scenes.cell_name(W, H, fx), f"1x{SWEEP_FRAMES}", [(0, SWEEP_FRAMES)]))
    out.append(("room640x480", f"1x{SWEEP_FRAMES}", [(0, SWEEP_FRAMES)]))
    return out


def write_calls(only=None):
    table = {}
    if os.path.exists(CALLS_PATH):
        with open(CALLS_PATH) as fh:
            table = json.load(fh)
    for name, split, calls in bench_splits():
        if only and name not in only:
            continue
        if split in table.get(name, {}):
            continue
        table.setdefault(name, {})[split] = call_counts(name, calls)
        with open(CALLS_PATH, "w") as fh:
            json.dump({"written_by": "tests/golden/make_golden.py calls (oracle only)", **{
                k: v for k, v in table.items() if k != "written_by"}}, fh, indent=1)
    print("wrote", CALLS_PATH)


def main(argv):
    if argv[:1] == ["calls"]:
        write_calls(argv[1:] or None)
        return
    if argv == ["sweep"]:
        # the sweep cells (the 640 x 480 cell is room640x480's first frames)
        names = [(scenes.cell_name(W, H, fx), SWEEP_FRAMES) for _, W, H, fx in scenes.SWEEP_CELLS
                 if (W, H) != (640, 480)]
    else:
        names = [(n, None) for n in (argv or ["room640x480", "cube640x480", "spherewall320x240", "plane64x48"])]
    for name, n_frames in names:
        out = make_counts(name, n_frames)
        path = os.path.join(HERE, f"{name}_counts.json")
        with open(path, "w") as fh:
            json.dump(out, fh, indent=1)
        print("wrote", path)


if __name__ == "__main__":
    main(sys.argv[1:])
