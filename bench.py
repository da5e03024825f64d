"""Benchmark of the integrate path (allocate + update) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload room640x480]

A step integrates the whole 100-frame, 640 x 480 room sequence into a
freshly reset volume, in calls of at most `--batch` frames (one allocate
launch and one update over a call's frames; the result equals
frame-by-frame integration);
inputs are resident in device memory before timing starts.  Timing is gated
on parity: the run first checks the volume against the oracle's stored
counts for the same seeded frames.  Per-call durations come from HIP events
recorded on the launch stream around every allocate and update call; per
kernel durations from the events the library records around each of its
kernels on the same stream (tsdf_set_kernel_timing), in separate steps of
the same work after the timed ones.  Prints one JSON line.

Rooflines.  The update kernel is HBM-bound; its algorithmic bytes per
frame (per frame counts from the oracle) are
  update    7 P + 16 B_t + 40 U
and those of the allocate stage
  allocate  4 P + 16 B_t + 16 B_n
with P pixels (depth 4 B, colour 3 B per pixel), B_t blocks touched (one
16-byte table entry read), B_n new blocks (one entry written), U distinct
voxels touched (five floats read and written).  The allocate kernel walks
every cell of every band: it is bound by vector ALU issue, and its
algorithmic work is counted in vector ops (ALU_OPS_PER_POINT per valid
point, ALU_OPS_PER_CELL per visited cell).  `roofline` is given for the
kernel that takes the most time; `path_roofline` puts the whole path
(allocate and update calls, every kernel in them) against HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
# Vector ALU issue of the chip for the walk's op mix (no FMA, no packed f32):
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic vector ops of allocate, counted from the walk's definition:
# per valid point the ray set-up (2 subtractions and 2 divisions for the
# ray, 6 for the band ends, 42 for the two ends' pose transform and
# scaling, 18 for the three axes' start cell, direction, reciprocal and
# first boundary) = 70; per visited cell the centre test (20: three centre
# coordinates, camera depth, difference, two comparisons) and the step
# (7: two comparisons for the axis, one for the end, the index step and
# the boundary's conversion, subtraction and product) = 27.
ALU_OPS_PER_POINT = 70
ALU_OPS_PER_CELL = 27


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    i = min(len(xs) - 1, max(0, int(round(q / 100.0 * (len(xs) - 1)))))
    return xs[i]


def load_counts(name):
    path = os.path.join(ROOT, "tests", "golden", f"{name}_counts.json")
    with open(path) as fh:
        return json.load(fh)


# HBM bytes per launch from hardware counters: rocprofv3 --pmc FETCH_SIZE,
# then WRITE_SIZE, each scaled by what it reads for a copy kernel of known
# size (the summaries under profiles/ give the commands and the factors).
# A figure holds only for the kernel sources it was taken on, so each entry
# carries their digest; after any change the field is null until re-measured.
MEASURED_TRAFFIC = {
    # (kernel, workload, most frames per call, update mode): (bytes per launch, source digest)
    # profiles/integrate_room640x480.md
    ("k_allocate", "room640x480", 128, "owner"): (1656772584, "01196f56cf83f2f5"),
    ("k_update_owner", "room640x480", 128, "owner"): (1950598219, "01196f56cf83f2f5"),
}


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ("tsdf_kernels.hip", "tsdf_device.hpp"):
        with open(os.path.join(ROOT, "hash_table_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, batch, mode):
    e = MEASURED_TRAFFIC.get((kernel, workload, batch, mode))
    if e is None or e[1] != kernel_source_digest():
        return None
    return e[0]


def split_calls(n, batch):
    """n frames in ceil(n / batch) calls of (nearly) equal size."""
    k = -(-n // batch)
    b = [round(i * n / k) for i in range(k + 1)]
    return [list(range(b[i], b[i + 1])) for i in range(k)]


def alloc_alu_ops(counts, calls):
    return sum(ALU_OPS_PER_POINT * counts["frames"][i]["points_valid"] +
               ALU_OPS_PER_CELL * counts["frames"][i]["cells_visited"] for c in calls for i in c)


def frame_bytes(fr):
    P = fr["pixels"]
    alloc = 4 * P + 16 * fr["blocks_touched"] + 16 * fr["blocks_new"]
    upd = 7 * P + 16 * fr["blocks_touched"] + 40 * fr["voxels_touched"]
    return alloc, upd


def microbench(torch, tsdf, stream):
    """Copy bandwidth and atomic / CAS rates (events on the launch stream)."""
    out = {}
    s = stream.cuda_stream

    def timed(fn, reps=5):
        ts = []
        for _ in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return statistics.median(ts[1:])

    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: tsdf.tsdf_mb_copy(src.data_ptr(), dst.data_ptr(), nbytes, s))
    out["copy_GBps"] = round(2 * nbytes / t / 1e9, 1)
    del src, dst
    n = 1 << 28                                     # 1 GiB of floats
    buf = torch.zeros(n, dtype=torch.float32, device="cuda")
    ops = 1 << 28
    for name, pat in (("coalesced", tsdf.MB_COALESCED), ("block_row", tsdf.MB_BLOCK_ROW),
                      ("random", tsdf.MB_RANDOM), ("same_wave", tsdf.MB_SAME_WAVE)):
        t = timed(lambda: tsdf.tsdf_mb_atomic_add_f32(buf.data_ptr(), n, ops, pat, 7, s))
        out[f"atomic_add_f32_{name}_Gops"] = round(ops / t / 1e9, 2)
    del buf
    n = 1 << 24
    cbuf = torch.zeros(n, dtype=torch.int64, device="cuda")
    ops = 1 << 26
    t = timed(lambda: tsdf.tsdf_mb_cas_u64(cbuf.data_ptr(), n, ops, 3, s))
    out["cas_u64_random_Gops"] = round(ops / t / 1e9, 2)
    del cbuf
    # LDS atomics, lane operations per clock per CU (256 CUs at 2.4 GHz)
    grid, iters = 256 * 8, 4096
    sink = torch.zeros(grid, dtype=torch.float32, device="cuda")
    for tname, ty in (("u32", tsdf.MB_LDS_U32), ("f32", tsdf.MB_LDS_F32), ("u64", tsdf.MB_LDS_U64)):
        for pname, pat in (("distinct", tsdf.MB_LDS_DISTINCT), ("random", tsdf.MB_LDS_RANDOM),
                           ("groups8", tsdf.MB_LDS_GROUPS)):
            t = timed(lambda: tsdf.tsdf_mb_lds_atomic(ty, pat, grid, iters, sink.data_ptr(), s), reps=3)
            out[f"lds_add_{tname}_{pname}_per_clk_per_cu"] = round(grid * 256 * iters / t / 2.4e9 / 256, 2)
    del sink
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, n_frames):
    """The oracle, single-threaded, on the first n_frames of the workload."""
    import oracle
    oracle.build()
    frames = [wl.frame(i) for i in range(n_frames)]
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity)
    t0 = time.perf_counter()
    for f in frames:
        o.integrate(f)
    dt = time.perf_counter() - t0
    tot = o.totals()
    return {
        "value": round(tot["points_valid"] / dt, 1),
        "unit": "points/s",
        "voxel_updates_per_s": round(tot["voxel_updates"] / dt, 1),
        "cores": 1,
        "host_cores": os.cpu_count(),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": f"first {n_frames} of {wl.n_frames} frames ({tot['points_valid']} points), {dt:.1f} s",
    }


def sweep(args, torch, tsdf, scenes, stream):
    """The paper's two opposite sweep axes on the room scene: point count at
    fixed geometry (fx proportional to the image width) and extent at fixed
    angular resolution (fx fixed).  Each cell integrates the scene's first 16
    frames in one batched call into a freshly reset volume; the first call is
    the parity gate against the oracle's stored counts for the same frames,
    then `--sweep-reps` calls are timed (HIP events around allocate and
    update, reset outside the windows).  Returns one record per cell."""
    sh = stream.cuda_stream
    cells = []
    for axis, W, H, fx in scenes.SWEEP_CELLS:
        name = scenes.cell_name(W, H, fx) if (W, H, fx) != (640, 480, 525.0) else "room640x480"
        wl = scenes.workload(name)
        counts = load_counts(name)
        n = 16
        host = [wl.frame(i) for i in range(n)]
        for i in (0, n - 1):
            if scenes.frame_digest([host[i]]) != counts["frames"][i]["sha256"]:
                raise SystemExit(f"{name}: generated frames differ from the stored oracle counts")
        fr = counts["frames"][:n]
        want = {"blocks": fr[-1]["blocks_total"], "voxel_updates": sum(f["voxel_updates"] for f in fr),
                "points_valid": sum(f["points_valid"] for f in fr)}
        frames = [tsdf.DeviceFrame(f) for f in host]
        vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, wl.table_entries,
                          max_batch_pixels=n * W * H)
        arr = tsdf.frame_array([f.desc for f in frames])
        tsdf.tsdf_integrate_batch(vol.handle, arr, sh, n=n)
        st = vol.stats()
        gate = {k: st["pool_used" if k == "blocks" else k] == v for k, v in want.items()}
        gate["no_loss"] = st["pool_overflow"] == st["table_full"] == st["update_misses"] == st["walk_guard"] == 0
        if not all(gate.values()):
            raise SystemExit(f"sweep cell {name}: parity gate failed {gate}")
        ta, tu = [], []
        for r in range(args.sweep_reps + 1):
            vol.reset()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            tsdf.tsdf_allocate_batch(vol.handle, arr, sh, n=n)
            e[1].record(stream)
            tsdf.tsdf_update_batch(vol.handle, arr, sh, n=n)
            e[2].record(stream)
            e[2].synchronize()
            if r:                                   # the first repetition warms up
                ta.append(e[0].elapsed_time(e[1]) * 1e-3)
                tu.append(e[1].elapsed_time(e[2]) * 1e-3)
        tt = [a + b for a, b in zip(ta, tu)]
        ba = sum(frame_bytes(f)[0] for f in fr)
        bu = sum(frame_bytes(f)[1] for f in fr)
        med = statistics.median
        cell = {"axis": axis, "workload": name, "width": W, "height": H, "fx": fx, "frames": n,
                "points": want["points_valid"], "voxel_updates": want["voxel_updates"], "blocks": want["blocks"],
                "voxel_updates_per_block_touch": round(want["voxel_updates"] / sum(f["blocks_touched"] for f in fr), 1),
                "reps": len(tt),
                "allocate_us": {"median": round(1e6 * med(ta), 1), "p95": round(1e6 * pct(ta, 95), 1),
                                "p99": round(1e6 * pct(ta, 99), 1)},
                "update_us": {"median": round(1e6 * med(tu), 1), "p95": round(1e6 * pct(tu, 95), 1),
                              "p99": round(1e6 * pct(tu, 99), 1)},
                "allocate_points_per_s": round(want["points_valid"] / med(ta), 1),
                "update_points_per_s": round(want["points_valid"] / med(tu), 1),
                "points_per_s": round(want["points_valid"] / med(tt), 1),
                "voxel_updates_per_s": round(want["voxel_updates"] / med(tt), 1),
                "path_GBps": round((ba + bu) / med(tt) / 1e9, 1),
                "path_hbm_frac": round((ba + bu) / med(tt) / 1e9 / HBM_PEAK_GBS, 4),
                "parity_gate": gate}
        log(f"[sweep] {axis:6s} {name:22s} alloc {cell['allocate_us']['median']:8.1f} us  "
            f"update {cell['update_us']['median']:8.1f} us  {cell['points_per_s'] / 1e9:6.2f} G points/s  "
            f"path {100 * cell['path_hbm_frac']:5.1f} % of HBM")
        cells.append(cell)
        del vol, frames
        torch.cuda.empty_cache()
    return cells


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="room640x480")
    ap.add_argument("--cpu-frames", type=int, default=100, help="frames of the workload the oracle integrates")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-microbench", action="store_true")
    ap.add_argument("--no-events", action="store_true", help="time whole steps only")
    ap.add_argument("--mode", default="owner", choices=["owner", "rays"], help="update organisation")
    ap.add_argument("--batch", type=int, default=128,
                    help="most frames per integrate call (1..128); the step's frames are split into equal calls")
    ap.add_argument("--no-variant", action="store_true", help="skip timing the per-frame variants")
    ap.add_argument("--sweep", action="store_true",
                    help="also run the sweep cells (point count at fixed geometry, extent at fixed "
                         "angular resolution), each gated on the oracle's stored counts")
    ap.add_argument("--sweep-reps", type=int, default=20, help="timed calls per sweep cell")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see the sharding note in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    from hash_table_amd import scenes, tsdf
    tsdf.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    wl = scenes.workload(args.workload)
    counts = load_counts(args.workload)
    log(f"generating {wl.n_frames} frames of {wl.name}")
    host_frames = [wl.frame(i) for i in range(wl.n_frames)]
    for i in (0, wl.n_frames - 1):
        if scenes.frame_digest([host_frames[i]]) != counts["frames"][i]["sha256"]:
            raise SystemExit("generated frames differ from the stored oracle counts")
    frames = [tsdf.DeviceFrame(f) for f in host_frames]
    tot = counts["totals"]
    pts = tot["points_valid"]
    vox = tot["voxel_updates"]

    def measure(mode, batch, steps, warmup, use_events):
        """Parity gate, then `steps` timed steps; returns (wall seconds,
        per-call allocate and update seconds, frame lists per call, stats, gate)."""
        vol = tsdf.Volume(wl.voxel_size, wl.trunc, wl.pool_capacity, wl.table_entries, update_mode=mode,
                          max_batch_pixels=batch * wl.width * wl.height)
        calls = split_calls(len(frames), batch)
        arrays = [tsdf.frame_array([frames[i].desc for i in c]) for c in calls]
        torch.cuda.synchronize()
        for arr, c in zip(arrays, calls):      # parity gate: one full pass vs the oracle's counts
            tsdf.tsdf_integrate_batch(vol.handle, arr, sh, n=len(c))
        st = vol.stats()
        gate = {
            "blocks": st["pool_used"] == tot["blocks"],
            "voxel_updates": st["voxel_updates"] == tot["voxel_updates"],
            "points_valid": st["points_valid"] == tot["points_valid"],
            "no_loss": st["pool_overflow"] == st["table_full"] == st["update_misses"] == st["walk_guard"] == 0,
            "no_rescans": st["fallback_blocks"] == 0,
        }
        log(f"[{mode} batch {batch}] parity gate", gate)
        if not all(gate.values()):
            raise SystemExit(f"parity gate failed ({mode}, batch {batch}): {gate}")
        ev = []

        def step(record):
            vol.reset()
            for arr, c in zip(arrays, calls):
                if record:
                    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                    e[0].record(stream)
                    tsdf.tsdf_allocate_batch(vol.handle, arr, sh, n=len(c))
                    e[1].record(stream)
                    tsdf.tsdf_update_batch(vol.handle, arr, sh, n=len(c))
                    e[2].record(stream)
                    ev.append((c, e))
                else:
                    tsdf.tsdf_integrate_batch(vol.handle, arr, sh, n=len(c))

        for _ in range(warmup):
            step(False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(use_events)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = vol.stats()
        kt = {}
        kt_steps = 0
        if use_events:
            # per-kernel durations from further steps of the same work with the
            # library's kernel events on (kept out of the timed steps above,
            # whose windows then hold only the kernels and their launch gaps)
            vol.set_kernel_timing(True)
            vol.kernel_times()
            kt_steps = max(2, steps // 2)
            for _ in range(kt_steps):
                step(False)
            torch.cuda.synchronize()
            kt = vol.kernel_times()
            vol.set_kernel_timing(False)
        t_alloc = [e[0].elapsed_time(e[1]) * 1e-3 for _, e in ev]
        t_upd = [e[1].elapsed_time(e[2]) * 1e-3 for _, e in ev]
        idx = [c for c, _ in ev]
        del vol
        torch.cuda.empty_cache()
        kt["_steps"] = kt_steps
        kt["_calls"] = calls
        return wall, t_alloc, t_upd, idx, st, gate, kt

    def kernel_report(t_alloc, t_upd, idx, steps):
        """Per-call durations -> throughput, algorithmic GB/s, per-frame latency."""
        b_alloc = [sum(frame_bytes(counts["frames"][i])[0] for i in c) for c in idx]
        b_upd = [sum(frame_bytes(counts["frames"][i])[1] for i in c) for c in idx]
        per_frame_a = [t / len(c) for t, c in zip(t_alloc, idx)]
        per_frame_u = [t / len(c) for t, c in zip(t_upd, idx)]
        ta, tu = sum(t_alloc), sum(t_upd)
        per = {
            "allocate": {"points_per_s": pts * steps / ta, "voxel_updates_per_s": vox * steps / ta,
                         "GBps": sum(b_alloc) / ta / 1e9, "us_per_frame_median": 1e6 * statistics.median(per_frame_a),
                         "us_per_frame_p95": 1e6 * pct(per_frame_a, 95),
                         "us_per_frame_p99": 1e6 * pct(per_frame_a, 99)},
            "update": {"points_per_s": pts * steps / tu, "voxel_updates_per_s": vox * steps / tu,
                       "GBps": sum(b_upd) / tu / 1e9, "us_per_frame_median": 1e6 * statistics.median(per_frame_u),
                       "us_per_frame_p95": 1e6 * pct(per_frame_u, 95),
                       "us_per_frame_p99": 1e6 * pct(per_frame_u, 99)},
            "integrate_kernels": {"points_per_s": pts * steps / (ta + tu),
                                  "voxel_updates_per_s": vox * steps / (ta + tu),
                                  "GBps": (sum(b_alloc) + sum(b_upd)) / (ta + tu) / 1e9},
            "calls": len(t_alloc),
        }
        for k in ("allocate", "update", "integrate_kernels"):
            per[k]["hbm_frac"] = per[k]["GBps"] / HBM_PEAK_GBS
            per[k] = {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in per[k].items()}
        return per, ta, tu, sum(b_alloc), sum(b_upd)

    use_events = not args.no_events
    wall, t_alloc, t_upd, idx, st, gate, ktimes = measure(args.mode, args.batch, args.steps, args.warmup, use_events)
    kt_steps, step_calls = ktimes.pop("_steps"), ktimes.pop("_calls")

    n_frames = wl.n_frames
    ms_per_step = wall / args.steps * 1e3
    out = {
        "metric": "integrated points/s and voxel-updates/s (allocate+update), % of HBM roofline",
        "value": round(pts * args.steps / wall, 1),
        "unit": "points/s",
        "voxel_updates_per_s": round(vox * args.steps / wall, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "frames_per_step": n_frames, "width": wl.width, "height": wl.height,
                   "voxel_size": wl.voxel_size, "trunc": wl.trunc, "pool_capacity": wl.pool_capacity,
                   "table_entries": wl.table_entries, "update_mode": args.mode, "max_frames_per_call": args.batch,
                   "calls_per_step": len(split_calls(wl.n_frames, args.batch)),
                   "points_per_step": pts, "voxel_updates_per_step": vox,
                   "step": "reset used pool + table, then allocate+update of all frames in equal calls"},
        "parity_gate": gate,
    }
    if use_events:
        per, ta, tu, ba, bu = kernel_report(t_alloc, t_upd, idx, args.steps)
        out["kernels"] = per
        # per-kernel durations: HIP events the library records on the launch
        # stream around each of its kernels (tsdf_set_kernel_timing)
        upd_kernel = "k_update_owner" if args.mode == "owner" else "k_update_rays"
        # algorithmic work of the kernel-timing steps (kt_steps steps of the same calls)
        ba_kt = kt_steps * sum(frame_bytes(counts["frames"][i])[0] for c in step_calls for i in c)
        bu_kt = kt_steps * sum(frame_bytes(counts["frames"][i])[1] for c in step_calls for i in c)
        alg = {"k_allocate": ba_kt, upd_kernel: bu_kt}
        kt = {}
        for name, v in sorted(ktimes.items(), key=lambda kv: -kv[1]["total_ms"]):
            e = {"launches": v["launches"], "avg_us": round(v["total_ms"] * 1e3 / v["launches"], 3),
                 "share_of_kernel_time": round(v["total_ms"] / sum(x["total_ms"] for x in ktimes.values()), 4)}
            if name in alg:
                e["algorithmic_GBps"] = round(alg[name] / (v["total_ms"] * 1e-3) / 1e9, 1)
            kt[name] = e
        out["kernel_times"] = kt
        # each stage kernel against the roof that binds it: allocate walks
        # every cell (integer/float vector work, no dense contraction), the
        # update moves the pool sums (HBM)
        ops = kt_steps * alloc_alu_ops(counts, step_calls)   # algorithmic vector ops, kernel-timing steps
        models = {"k_allocate": ("alu", ops / 1e12, ALU_PEAK_TOPS, "TOP/s"),
                  upd_kernel: ("hbm", bu_kt / 1e9, HBM_PEAK_GBS, "GB/s")}
        dom = max((k for k in models if k in ktimes), key=lambda k: ktimes[k]["total_ms"])
        bound, amount, peak, unit = models[dom]
        launches = ktimes[dom]["launches"]
        avg_s = ktimes[dom]["total_ms"] * 1e-3 / launches
        achieved = amount / launches / avg_s
        out["roofline"] = {"kernel": dom, "bound": bound, "achieved": round(achieved, 3 if bound == "alu" else 1),
                           "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                           "traffic": measured_traffic(dom, args.workload, args.batch, args.mode),
                           "algorithmic_per_launch": round(amount / launches * (1e12 if bound == "alu" else 1e9)),
                           "avg_launch_us": round(avg_s * 1e6, 3)}
        for k in models:
            if k in ktimes:
                b_, a_, p_, u_ = models[k]
                kt[k]["roof"] = {"bound": b_, "achieved": round(a_ / (ktimes[k]["total_ms"] * 1e-3), 3),
                                 "peak": p_, "unit": u_,
                                 "frac": round(a_ / (ktimes[k]["total_ms"] * 1e-3) / p_, 4)}
        # the whole path (allocate and update calls, every kernel in them)
        # against HBM: the paper's framing of the integrate step
        out["path_roofline"] = {"bound": "hbm", "achieved": per["integrate_kernels"]["GBps"], "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": per["integrate_kernels"]["hbm_frac"]}
    if not args.no_variant:
        out["variants"] = {}
        for mode, batch in (("owner", 1), ("rays", 1)):
            if (mode, batch) == (args.mode, args.batch):
                continue
            vs = max(1, args.steps // 2)
            w2, a2, u2, i2, _, g2, _ = measure(mode, batch, vs, 1, True)
            per2, *_ = kernel_report(a2, u2, i2, vs)
            out["variants"][f"{mode}_batch{batch}"] = {"points_per_s": round(pts * vs / w2, 1),
                                                       "ms_per_step": round(w2 / vs * 1e3, 4),
                                                       "kernels": per2, "parity_gate": g2}
    out["loss_counters"] = {k: st[k] for k in ("pool_overflow", "table_full", "update_misses", "walk_guard")}
    if not args.no_microbench:
        log("microbenchmarks")
        out["microbench"] = microbench(torch, tsdf, stream)
    if args.sweep:
        log("sweep cells")
        out["sweep"] = sweep(args, torch, tsdf, scenes, stream)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_frames} frames")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_frames)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
