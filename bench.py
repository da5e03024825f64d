"""Benchmark of the integrate path (allocate + update) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cells] [--sweep]

Headline.  A step integrates the whole 100-frame, 640 x 480 room sequence
into a freshly reset volume in calls of at most `--batch` frames (one call of
100: one allocate launch and one update over the call's frames; the result
equals frame-by-frame integration).  Inputs are resident in device memory
before timing starts; the step includes the volume reset.  Timing is gated
on parity: the run first checks the volume against the oracle's stored
counts for the same seeded frames.  W untimed warm-up steps, then exactly K
timed steps between two device synchronisations; `value` = valid points per
second over them.  Per-call durations come from HIP events on the launch
stream around every allocate and update call; per-kernel durations from the
events the library records around each of its kernels on the same stream
(tsdf_set_kernel_timing), in further steps of the same work after the
timed ones.

Rooflines (bytes are algorithmic: what the method must move, not what the
hardware moved; HBM peak 8.0 TB/s):
  * `roofline`: the kernel that takes the most time, with the per-frame
    bytes of the method for it, summed over the frames one launch covers:
      allocate  4 P + 16 B_t + 16 B_n     (depth; one table entry read per
                                            touched block, one written per new one)
      update    7 P + 16 B_t + 40 U       (depth and colour; entry; five
                                            floats read and written per voxel)
    P pixels, B_t / B_n / U the frame's distinct blocks, new blocks and
    distinct voxels (oracle counts, tests/golden/).  `roofline_alu` puts the
    same launch against the vector-ALU issue rate (256 CUs x 4 SIMDs x 16
    lanes x 2.4 GHz) with 20 operations per valid point and 15 per visited
    cell.
  * `path_roofline` and the per-stage figures: the compulsory bytes of the
    calls as launched -- a batched call reads and writes each block it
    touches once --
      allocate  4 P + 16 B_call + 16 B_new
      update    7 P + 16 B_call + 20 U_fresh + 40 U_old
    (B_call distinct blocks of the call, B_new the blocks it creates,
    U_fresh / U_old its distinct voxels in blocks it created / in older
    blocks: a fresh block is written without being read), from the oracle's
    per-call counts (tests/golden/calls.json), with the measured HBM
    traffic beside them where the counters were taken on the current
    kernels.

Cells.  Every configuration as its own parity-gated cell -- the plane, the
sphere-and-wall arc, the load-factor cells (0.1, 0.25, 0.5), the contention
cube, the 1280 x 720 room at its full 300 frames -- with allocate, update
and combined rates, their fraction of the compulsory-byte roofline, median /
p95 / p99 over the repetitions, and the device's clocks and temperatures
before and after each cell.  Variants (per-frame owner and ray-parallel
updates) run interleaved with the headline configuration in rotated order,
with a first-half / second-half drift check.  An exclusive-device check
(other processes holding the GPU) runs before the first GPU call.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
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
# Vector ALU issue of the chip (no FMA by the float contract, no packed f32):
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-operations/s.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic vector operations of the walk: about 20 per valid point (ray,
# band ends, pose transform, set-up of the three axes) and 15 per visited
# cell (centre test and step).
ALU_OPS_PER_POINT = 20
ALU_OPS_PER_CELL = 15


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    i = min(len(xs) - 1, max(0, int(round(q / 100.0 * (len(xs) - 1)))))
    return xs[i]


def dist(xs, scale=1e6, nd=1):
    """median / p95 / p99 (in scale units) and the repeat count."""
    return {"median": round(scale * statistics.median(xs), nd), "p95": round(scale * pct(xs, 95), nd),
            "p99": round(scale * pct(xs, 99), nd), "reps": len(xs)}


def load_counts(name):
    with open(os.path.join(ROOT, "tests", "golden", f"{name}_counts.json")) as fh:
        return json.load(fh)


def load_calls():
    with open(os.path.join(ROOT, "tests", "golden", "calls.json")) as fh:
        return json.load(fh)


# HBM bytes per launch from hardware counters: rocprofv3 --pmc FETCH_SIZE,
# then WRITE_SIZE, each scaled by what it reads for a copy kernel of known
# size (the summaries under profiles/ give the commands and the factors).
# A figure holds only for the kernel sources it was taken on, so each entry
# carries their digest; after any change the field is null until re-measured.
MEASURED_TRAFFIC = {
    # (kernel, workload, most frames per call, update mode): (bytes per launch, source digest)
    ("k_allocate", "room640x480", 128, "owner"): (1264350746, "05d6a1f3d953e27d"),
    ("k_place_items", "room640x480", 128, "owner"): (6606266, "05d6a1f3d953e27d"),
    ("k_place_segments", "room640x480", 128, "owner"): (260498753, "05d6a1f3d953e27d"),
    ("k_update_owner", "room640x480", 128, "owner"): (1392649738, "05d6a1f3d953e27d"),
}


def kernel_source_digest() -> str:
    """Digest of the integrate kernels' sources with comments and layout
    removed (a change of code, not of comments, invalidates the figures)."""
    import re
    h = hashlib.sha256()
    for name in ("tsdf_kernels.hip", "tsdf_device.hpp"):
        with open(os.path.join(ROOT, "hash_table_amd", "csrc", name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
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


# ---------------------------------------------------------------------------
# algorithmic bytes and operations
# ---------------------------------------------------------------------------
def frame_bytes(fr):
    """The method's per-frame bytes: (allocate, update)."""
    P = fr["pixels"]
    return (4 * P + 16 * fr["blocks_touched"] + 16 * fr["blocks_new"],
            7 * P + 16 * fr["blocks_touched"] + 40 * fr["voxels_touched"])


def call_bytes(c):
    """Compulsory bytes of one batched call: (allocate, update)."""
    P = c["pixels"]
    return (4 * P + 16 * c["blocks_touched"] + 16 * c["blocks_new"],
            7 * P + 16 * c["blocks_touched"] + 20 * c["voxels_fresh"] + 40 * c["voxels_old"])


def walk_ops(frames):
    return sum(ALU_OPS_PER_POINT * f["points_valid"] + ALU_OPS_PER_CELL * f["cells_visited"] for f in frames)


# ---------------------------------------------------------------------------
# the device: exclusivity, clocks, temperatures (sysfs; no GPU call)
# ---------------------------------------------------------------------------
TELEMETRY = True      # --no-telemetry: no amd-smi (e.g. under a profiler, whose preload reaches child processes)


def _amd_smi(*args):
    """amd-smi's JSON output (run as a child process), or None."""
    import subprocess
    if not TELEMETRY:
        return None
    try:
        out = subprocess.run(["amd-smi", *args, "--json"], capture_output=True, text=True, timeout=30)
        text = out.stdout
        starts = [i for i in (text.find("{"), text.find("[")) if i >= 0]   # (a warning line may come first)
        return json.loads(text[min(starts):]) if out.returncode == 0 and starts else None
    except (OSError, ValueError, subprocess.SubprocessError):
        return None


def device_holders():
    """Other processes holding the GPU: amd-smi's process list, and the KFD
    process directory where sysfs has one.  None if neither can be read."""
    found, seen = [], False
    data = _amd_smi("process")
    if isinstance(data, list):
        seen = True
        for gpu in data:
            for p in gpu.get("process_list", []):
                info = p.get("process_info")
                if isinstance(info, dict) and info.get("pid") not in (None, os.getpid()):
                    found.append({"pid": info.get("pid"), "name": info.get("name")})
    d = "/sys/class/kfd/kfd/proc"
    if os.path.isdir(d):
        seen = True
        for q in os.listdir(d):
            if q.isdigit() and int(q) != os.getpid() and all(f["pid"] != int(q) for f in found):
                found.append({"pid": int(q), "name": None})
    return found if seen else None


def _val(x):
    return x.get("value") if isinstance(x, dict) and isinstance(x.get("value"), (int, float)) else None


def telemetry():
    """Clocks (MHz), temperatures (C) and power (W) of GPU 0 from amd-smi
    (graphics clock per XCD as min / max), or {"error": ...}."""
    data = _amd_smi("metric", "-c", "-t", "-p")
    try:
        g = data["gpu_data"][0]
    except (TypeError, KeyError, IndexError):
        return {"error": "amd-smi metric unavailable"}
    out = {}
    clk = g.get("clock", {})
    gfx = [_val(v.get("clk")) for k, v in clk.items() if k.startswith("gfx") and isinstance(v, dict)]
    gfx = [x for x in gfx if x is not None]
    if gfx:
        out["gfx_clk_MHz"] = {"min": min(gfx), "max": max(gfx)}
    for k, v in clk.items():
        if k.startswith("mem") and isinstance(v, dict) and _val(v.get("clk")) is not None:
            out["mem_clk_MHz"] = _val(v.get("clk"))
    t = g.get("temperature", {})
    for k in ("edge", "hotspot", "mem"):
        if _val(t.get(k)) is not None:
            out[f"temp_{k}_C"] = _val(t.get(k))
    p = g.get("power", {})
    if _val(p.get("socket_power")) is not None:
        out["socket_power_W"] = _val(p.get("socket_power"))
    return out or {"error": "amd-smi metric had no readable fields"}


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------
class Runner:
    def __init__(self, torch, tsdf, stream):
        self.torch, self.tsdf, self.stream = torch, tsdf, stream
        self.sh = stream.cuda_stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def volume(self, wl_vs, wl_tr, cap, table, mode, batch_pixels, probe_limit=0):
        return self.tsdf.Volume(wl_vs, wl_tr, cap, table, update_mode=mode, max_batch_pixels=batch_pixels,
                                probe_limit=probe_limit)

    def integrate_calls(self, vol, arrays, calls, record=None):
        """One pass over the calls (allocate + update each); with `record`,
        HIP events around each allocate and update are appended to it."""
        tsdf, sh = self.tsdf, self.sh
        for arr, c in zip(arrays, calls):
            if record is None:
                tsdf.tsdf_integrate_batch(vol.handle, arr, sh, n=len(c))
            else:
                e0 = self.event()
                tsdf.tsdf_allocate_batch(vol.handle, arr, sh, n=len(c))
                e1 = self.event()
                tsdf.tsdf_update_batch(vol.handle, arr, sh, n=len(c))
                e2 = self.event()
                record.append((c, e0, e1, e2))

    @staticmethod
    def call_times(record):
        a = [e0.elapsed_time(e1) * 1e-3 for _, e0, e1, _ in record]
        u = [e1.elapsed_time(e2) * 1e-3 for _, _, e1, e2 in record]
        return a, u


def gate(st, want):
    g = {
        "blocks": st["pool_used"] == want["blocks"],
        "voxel_updates": st["voxel_updates"] == want["voxel_updates"],
        "points_valid": st["points_valid"] == want["points_valid"],
        "no_loss": st["pool_overflow"] == st["table_full"] == st["update_misses"] == st["walk_guard"] == 0,
        "no_rescans": st["fallback_blocks"] == 0,
    }
    return g


def cell_run(R, name, host_frames, vs, tr, cap, table, calls, frame_counts, call_counts, reps, warmup=1,
             mode="owner"):
    """A parity-gated cell: one pass against the stored counts, then `reps`
    timed passes (each into a freshly reset volume; the reset is outside the
    allocate / update windows).  Returns the cell's record."""
    torch, tsdf = R.torch, R.tsdf
    t_before = telemetry()
    frames = [tsdf.DeviceFrame(f) for f in host_frames]
    batch_px = max(sum(host_frames[i].width * host_frames[i].height for i in c) for c in calls)
    vol = R.volume(vs, tr, cap, table, mode, batch_px)
    arrays = [tsdf.frame_array([frames[i].desc for i in c]) for c in calls]
    R.integrate_calls(vol, arrays, calls)
    st = vol.stats()
    want = {"blocks": frame_counts[-1]["blocks_total"],
            "voxel_updates": sum(f["voxel_updates"] for f in frame_counts),
            "points_valid": sum(f["points_valid"] for f in frame_counts)}
    g = gate(st, want)
    if not all(g.values()):
        raise SystemExit(f"cell {name}: parity gate failed {g}")
    for _ in range(warmup):
        vol.reset()
        R.integrate_calls(vol, arrays, calls)
    ta, tu = [], []
    for _ in range(reps):
        vol.reset()
        rec = []
        R.integrate_calls(vol, arrays, calls, rec)
        torch.cuda.synchronize()
        a, u = R.call_times(rec)
        ta.append(sum(a))
        tu.append(sum(u))
    tt = [a + u for a, u in zip(ta, tu)]
    pts, vox = want["points_valid"], want["voxel_updates"]
    ba = sum(call_bytes(c)[0] for c in call_counts)
    bu = sum(call_bytes(c)[1] for c in call_counts)
    med = statistics.median
    rec = {
        "workload": name, "frames": len(host_frames), "calls": len(calls),
        "pool_capacity": cap, "table_entries": table, "blocks": want["blocks"],
        "load_factor": round(want["blocks"] / table, 4),
        "points": pts, "voxel_updates": vox, "update_mode": mode,
        "allocate_us": dist(ta), "update_us": dist(tu), "integrate_us": dist(tt),
        "allocate": {"points_per_s": round(pts / med(ta), 1), "voxel_updates_per_s": round(vox / med(ta), 1),
                     "compulsory_bytes": ba, "hbm_frac": round(ba / med(ta) / 1e9 / HBM_PEAK_GBS, 5)},
        "update": {"points_per_s": round(pts / med(tu), 1), "voxel_updates_per_s": round(vox / med(tu), 1),
                   "compulsory_bytes": bu, "hbm_frac": round(bu / med(tu) / 1e9 / HBM_PEAK_GBS, 5)},
        "integrate": {"points_per_s": round(pts / med(tt), 1), "voxel_updates_per_s": round(vox / med(tt), 1),
                      "compulsory_bytes": ba + bu, "hbm_frac": round((ba + bu) / med(tt) / 1e9 / HBM_PEAK_GBS, 5)},
        "probe_max": st["probe_max"],
        "parity_gate": g,
        "telemetry": {"before": t_before, "after": telemetry()},
    }
    log(f"[cell] {name:24s} {len(calls)} call(s)  alloc {rec['allocate_us']['median']:9.1f} us  "
        f"update {rec['update_us']['median']:9.1f} us  {rec['integrate']['points_per_s'] / 1e9:6.2f} G points/s")
    del vol, frames, arrays
    torch.cuda.empty_cache()
    return rec


def _render_range(args):
    name, a, b = args
    from hash_table_amd import scenes
    wl = scenes.workload(name)
    return a, [wl.frame(i) for i in range(a, b)]


def render_frames(name, n, workers=8):
    """Frames [0, n) of a workload, rendered in worker processes (spawned:
    they load no GPU library)."""
    import multiprocessing as mp
    b = [round(i * n / workers) for i in range(workers + 1)]
    jobs = [(name, b[i], b[i + 1]) for i in range(workers) if b[i + 1] > b[i]]
    out = {}
    with mp.get_context("spawn").Pool(len(jobs)) as pool:
        for a, fr in pool.imap_unordered(_render_range, jobs):
            for i, f in enumerate(fr):
                out[a + i] = f
    return [out[i] for i in range(n)]


def config_cells(R, scenes, host_room, args):
    """Configurations 1, 2, 4 (load factors and the cube) and 5."""
    calls_tab = load_calls()
    cells = []

    def check_inputs(name, frames, counts):
        for i in sorted({0, len(frames) - 1}):
            if scenes.frame_digest([frames[i]]) != counts["frames"][i]["sha256"]:
                raise SystemExit(f"{name}: generated frames differ from the stored oracle counts")

    for name in ("plane64x48", "spherewall320x240", "cube640x480"):
        wl = scenes.workload(name)
        counts = load_counts(name)
        host = [wl.frame(i) for i in range(wl.n_frames)]
        check_inputs(name, host, counts)
        split = scenes.BENCH_CALLS[name]
        calls = [list(range(a, b)) for a, b in split]
        cc = calls_tab[name][f"{len(split)}x{split[0][1] - split[0][0]}"]
        rec = cell_run(R, name, host, wl.voxel_size, wl.trunc, wl.pool_capacity, wl.table_entries, calls,
                       counts["frames"], cc, reps=args.cell_reps)
        rec["config"] = {"plane64x48": 1, "spherewall320x240": 2, "cube640x480": "4-cube"}[name]
        cells.append(rec)
    # load-factor cells: prefixes of the room with a pool of 2^k blocks
    wl = scenes.workload("room640x480")
    counts = load_counts("room640x480")
    totals = [f["blocks_total"] for f in counts["frames"]]
    for lf in scenes.LOAD_FACTORS:
        cap, n, achieved = scenes.load_factor_cell(totals, lf)
        cc = calls_tab["room640x480"][f"prefix{n}"]
        rec = cell_run(R, f"room640x480_lf{lf}", host_room[:n], wl.voxel_size, wl.trunc, cap, 2 * cap,
                       [list(range(n))], counts["frames"][:n], cc, reps=args.cell_reps)
        rec["config"] = f"4-lf{lf}"
        rec["load_factor_target"] = lf
        cells.append(rec)
    if not args.no_room1280:
        name = "room1280x720"
        wl = scenes.workload(name)
        counts = load_counts(name)
        log(f"rendering {wl.n_frames} frames of {name}")
        host = render_frames(name, wl.n_frames)
        check_inputs(name, host, counts)
        split = scenes.BENCH_CALLS[name]
        calls = [list(range(a, b)) for a, b in split]
        cc = calls_tab[name][f"{len(split)}x{split[0][1] - split[0][0]}"]
        rec = cell_run(R, name, host, wl.voxel_size, wl.trunc, wl.pool_capacity, wl.table_entries, calls,
                       counts["frames"], cc, reps=max(3, args.cell_reps // 2))
        rec["config"] = 5
        cells.append(rec)
        del host
    return cells


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
    n = 1 << 28
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


def cpu_baseline(wl, host_frames, n_frames):
    """The oracle, single-threaded, on the first n_frames of the workload."""
    import oracle
    oracle.build()
    o = oracle.Oracle(wl.voxel_size, wl.trunc, wl.pool_capacity)
    t0 = time.perf_counter()
    for f in host_frames[:n_frames]:
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
        "sample": f"first {n_frames} of {wl.n_frames} frames of {wl.name} ({tot['points_valid']} points), "
                  f"{dt:.1f} s on one thread",
    }


def sweep(R, scenes, args):
    """The paper's two sweep axes on the room scene (point count at fixed
    geometry, extent at fixed angular resolution), 16 frames per cell in one
    batched call, each cell parity-gated on the stored counts."""
    calls_tab = load_calls()
    cells = []
    for axis, W, H, fx in scenes.SWEEP_CELLS:
        name = scenes.cell_name(W, H, fx) if (W, H, fx) != (640, 480, 525.0) else "room640x480"
        wl = scenes.workload(name)
        counts = load_counts(name)
        n = 16
        host = [wl.frame(i) for i in range(n)]
        if scenes.frame_digest([host[n - 1]]) != counts["frames"][n - 1]["sha256"]:
            raise SystemExit(f"{name}: generated frames differ from the stored oracle counts")
        rec = cell_run(R, name, host, wl.voxel_size, wl.trunc, wl.pool_capacity, wl.table_entries,
                       [list(range(n))], counts["frames"][:n], calls_tab[name]["1x16"], reps=args.sweep_reps)
        rec["axis"] = axis
        rec["fx"] = fx
        cells.append(rec)
    return cells


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--batch", type=int, default=128,
                    help="most frames per integrate call (1..128); the step's frames are split into equal calls")
    ap.add_argument("--rounds", type=int, default=6, help="rounds of the rotated headline / variant comparison")
    ap.add_argument("--cell-reps", type=int, default=10, help="timed repetitions per configuration cell")
    ap.add_argument("--no-cells", action="store_true", help="skip the per-configuration cells")
    ap.add_argument("--no-room1280", action="store_true", help="skip the 1280 x 720 room cell")
    ap.add_argument("--no-variants", action="store_true", help="skip the rotated variant comparison")
    ap.add_argument("--no-microbench", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frames", type=int, default=100, help="frames of the room the oracle integrates")
    ap.add_argument("--require-exclusive", action="store_true",
                    help="refuse to run when another process holds the GPU")
    ap.add_argument("--sweep", action="store_true", help="also run the sweep cells (gated on stored counts)")
    ap.add_argument("--sweep-reps", type=int, default=20)
    ap.add_argument("--no-telemetry", action="store_true",
                    help="no amd-smi calls (exclusivity, clocks, temperatures), e.g. under rocprofv3")
    args = ap.parse_args()
    global TELEMETRY
    TELEMETRY = not args.no_telemetry
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the sharding design is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    # before any GPU call: is the device ours alone?
    holders = device_holders()
    exclusive = {"checked": holders is not None, "other_processes": holders,
                 "exclusive": (holders == []) if holders is not None else None}
    if holders:
        log(f"warning: other processes hold the GPU: {holders}")
        if args.require_exclusive:
            raise SystemExit("the device is not exclusive (--require-exclusive)")
    t_start = telemetry()

    import torch
    from hash_table_amd import scenes, tsdf
    tsdf.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    R = Runner(torch, tsdf, stream)

    wl = scenes.workload("room640x480")
    counts = load_counts(wl.name)
    calls_tab = load_calls()
    log(f"generating {wl.n_frames} frames of {wl.name}")
    host_room = [wl.frame(i) for i in range(wl.n_frames)]
    for i in (0, wl.n_frames - 1):
        if scenes.frame_digest([host_room[i]]) != counts["frames"][i]["sha256"]:
            raise SystemExit("generated frames differ from the stored oracle counts")
    frames = [tsdf.DeviceFrame(f) for f in host_room]
    tot = counts["totals"]
    pts, vox = tot["points_valid"], tot["voxel_updates"]

    def setup(mode, batch):
        vol = R.volume(wl.voxel_size, wl.trunc, wl.pool_capacity, wl.table_entries, mode,
                       batch * wl.width * wl.height)
        calls = split_calls(len(frames), batch)
        arrays = [tsdf.frame_array([frames[i].desc for i in c]) for c in calls]
        R.integrate_calls(vol, arrays, calls)           # parity gate: one full pass vs the stored counts
        g = gate(vol.stats(), {"blocks": tot["blocks"], "voxel_updates": vox, "points_valid": pts})
        log(f"[{mode} batch {batch}] parity gate", g)
        if not all(g.values()):
            raise SystemExit(f"parity gate failed ({mode}, batch {batch}): {g}")
        return vol, calls, arrays, g

    def step(vol, calls, arrays, record=None):
        vol.reset()
        R.integrate_calls(vol, arrays, calls, record)

    # ---- headline: K timed steps of the main configuration ----
    vol, calls, arrays, g_main = setup("owner", args.batch)
    for _ in range(args.warmup):
        step(vol, calls, arrays)
    rec_main = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(vol, calls, arrays, rec_main)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st_main = vol.stats()
    t_alloc, t_upd = R.call_times(rec_main)
    # per-kernel durations: the library's events on the launch stream, in
    # further steps of the same work
    vol.set_kernel_timing(True)
    vol.kernel_times()
    kt_steps = max(2, args.steps // 2)
    for _ in range(kt_steps):
        step(vol, calls, arrays)
    torch.cuda.synchronize()
    ktimes = vol.kernel_times()
    vol.set_kernel_timing(False)

    ms_per_step = wall / args.steps * 1e3
    split = f"{len(calls)}x{len(calls[0])}"
    cc = calls_tab[wl.name].get(split)
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
        "dtype_note": "f32 walk and pool sums; within a call the owner update sums a block's terms in LDS as "
                      "integers (signed distance in 2^-24 units, colour bytes), converted to f32 once",
        "data": "synthetic",
        "config": {"workload": wl.name, "frames_per_step": wl.n_frames, "width": wl.width, "height": wl.height,
                   "voxel_size": wl.voxel_size, "trunc": wl.trunc, "pool_capacity": wl.pool_capacity,
                   "table_entries": wl.table_entries, "update_mode": "owner", "max_frames_per_call": args.batch,
                   "calls_per_step": len(calls), "points_per_step": pts, "voxel_updates_per_step": vox,
                   "step": "reset used pool + table, then allocate+update of all frames in equal calls"},
        "parity_gate": g_main,
        "device": {"exclusive": exclusive, "telemetry_start": t_start},
    }
    ta, tu = sum(t_alloc), sum(t_upd)
    frames_of = [counts["frames"][i] for c in calls for i in c]
    # per-frame bytes of the method, and the calls' compulsory bytes
    fb_a = sum(frame_bytes(f)[0] for f in frames_of)
    fb_u = sum(frame_bytes(f)[1] for f in frames_of)
    cb_a = sum(call_bytes(c)[0] for c in cc) if cc else None
    cb_u = sum(call_bytes(c)[1] for c in cc) if cc else None
    stages = {}
    for key, t, b in (("allocate", ta, cb_a), ("update", tu, cb_u),
                      ("integrate", ta + tu, (cb_a + cb_u) if cc else None)):
        d = {"points_per_s": round(pts * args.steps / t, 1), "voxel_updates_per_s": round(vox * args.steps / t, 1),
             "us_per_step": dist([x for x in (t_alloc if key == "allocate" else t_upd if key == "update" else
                                             [a + u for a, u in zip(t_alloc, t_upd)])])}
        if b is not None:
            d["compulsory_bytes_per_step"] = b
            d["hbm_frac"] = round(b * args.steps / t / 1e9 / HBM_PEAK_GBS, 5)
        stages[key] = d
    out["stages"] = stages
    kt = {}
    total_ms = sum(x["total_ms"] for x in ktimes.values())
    for name, v in sorted(ktimes.items(), key=lambda kv: -kv[1]["total_ms"]):
        kt[name] = {"launches": v["launches"], "avg_us": round(v["total_ms"] * 1e3 / v["launches"], 3),
                    "share_of_kernel_time": round(v["total_ms"] / total_ms, 4)}
    out["kernel_times"] = kt
    # roofline of the dominant kernel against HBM, the ALU model beside it.
    # Allocate: the method's per-frame bytes over the frames its launch
    # covers.  Update: a batched call reads and writes each touched voxel once
    # for all its frames, so its per-frame bytes (every frame's own
    # read-modify-write) would exceed what the launch must move; it takes the
    # call's compulsory bytes instead.
    per_launch = {"k_allocate": fb_a, "k_update_owner": cb_u if cc else None}
    dom = max((k for k in per_launch if k in ktimes and per_launch[k] is not None),
              key=lambda k: ktimes[k]["total_ms"])
    launches = ktimes[dom]["launches"]
    avg_s = ktimes[dom]["total_ms"] * 1e-3 / launches
    launches_per_step = len(calls)                    # launches of each kernel per step
    alg = per_launch[dom] / launches_per_step
    achieved = alg / avg_s / 1e9
    out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                       "traffic": measured_traffic(dom, wl.name, args.batch, "owner"),
                       "algorithmic_bytes_per_launch": int(alg), "avg_launch_us": round(avg_s * 1e6, 3),
                       "bytes": "allocate: per frame 4 P + 16 B_t + 16 B_n, summed over the launch's frames; "
                                "update: per call 7 P + 16 B_call + 20 U_fresh + 40 U_old"}
    ops = walk_ops(frames_of) / launches_per_step
    out["roofline_alu"] = {"kernel": "k_allocate", "bound": "alu",
                           "achieved": round(ops / (ktimes["k_allocate"]["total_ms"] * 1e-3 /
                                                    ktimes["k_allocate"]["launches"]) / 1e12, 3),
                           "peak": round(ALU_PEAK_TOPS, 2), "unit": "TOP/s",
                           "ops": f"{ALU_OPS_PER_POINT} per valid point + {ALU_OPS_PER_CELL} per visited cell",
                           "ops_per_launch": int(ops)}
    out["roofline_alu"]["frac"] = round(out["roofline_alu"]["achieved"] / ALU_PEAK_TOPS, 4)
    kernel_per_step = {k: v["total_ms"] / kt_steps * 1e-3 for k, v in ktimes.items()}
    if cc:
        for k, b in (("k_allocate", cb_a), ("k_update_owner", cb_u)):
            if k in ktimes:
                t = ktimes[k]["total_ms"] * 1e-3 / ktimes[k]["launches"]
                kt[k]["compulsory_bytes_per_launch"] = int(b / launches_per_step)
                kt[k]["compulsory_hbm_frac"] = round(b / launches_per_step / t / 1e9 / HBM_PEAK_GBS, 5)
        traffic = [measured_traffic(k, wl.name, args.batch, "owner")
                   for k in ("k_allocate", "k_place_items", "k_place_segments", "k_update_owner")]
        out["path_roofline"] = {
            "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "compulsory_bytes_per_step": cb_a + cb_u,
            "achieved": round((cb_a + cb_u) / (ms_per_step * 1e-3) / 1e9, 1),
            "frac": round((cb_a + cb_u) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
            "kernel_seconds_per_step": round(sum(kernel_per_step.values()), 6),
            # counter-measured HBM bytes of the step's allocate, placing and update kernels
            "measured_traffic_per_step": (sum(traffic) * launches_per_step) if None not in traffic else None,
            "bytes": "per call 4 P + 16 B_call + 16 B_new (allocate) + 7 P + 16 B_call + 20 U_fresh + 40 U_old "
                     "(update); time = the whole step (reset and launch gaps included)"}
        if out["path_roofline"]["measured_traffic_per_step"]:
            out["path_roofline"]["traffic_over_compulsory"] = round(
                out["path_roofline"]["measured_traffic_per_step"] / (cb_a + cb_u), 2)
    out["loss_counters"] = {k: st_main[k] for k in ("pool_overflow", "table_full", "update_misses", "walk_guard")}
    out["device"]["telemetry_after_headline"] = telemetry()
    if TELEMETRY:
        # the clocks with the GPU at work: steps of the headline queued for
        # half a second (the clocks ramp up), then amd-smi run (a child
        # process, in a thread) while this thread keeps queueing them
        import threading
        sample = []
        th = threading.Thread(target=lambda: sample.append(telemetry()))
        n_load, t_load = 0, time.perf_counter()
        while time.perf_counter() - t_load < 0.5:
            step(vol, calls, arrays)
            n_load += 1
        th.start()
        while th.is_alive():
            step(vol, calls, arrays)
            n_load += 1
        torch.cuda.synchronize()
        out["device"]["telemetry_under_load"] = (dict(sample[0], steps_queued=n_load,
                                                      seconds=round(time.perf_counter() - t_load, 2))
                                                 if sample else None)

    # ---- the headline configuration and its variants, interleaved and rotated ----
    if not args.no_variants:
        variants = [("owner", args.batch), ("owner", 1), ("rays", 1)]
        setups = {v: (vol, calls, arrays) if v == ("owner", args.batch) else setup(*v)[:3] for v in variants}
        times = {v: [] for v in variants}
        clocks = []
        for r in range(args.rounds):
            order = variants[r % len(variants):] + variants[:r % len(variants)]
            for v in order:
                vv, cl, ar = setups[v]
                torch.cuda.synchronize()
                e0 = R.event()
                step(vv, cl, ar)
                e1 = R.event()
                e1.synchronize()
                times[v].append(e0.elapsed_time(e1) * 1e-3)
            clocks.append(telemetry())
        rot = {}
        for v, ts in times.items():
            h = len(ts) // 2                  # (one round: no halves to compare)
            first, second = (statistics.median(ts[:h]), statistics.median(ts[h:])) if h else (ts[0], ts[0])
            rot[f"{v[0]}_batch{v[1]}"] = {"step_ms": dist(ts, 1e3, 4), "points_per_s": round(pts / statistics.median(ts), 1),
                                          "first_half_ms": round(first * 1e3, 4), "second_half_ms": round(second * 1e3, 4),
                                          "drift": round(second / first - 1.0, 4)}
        out["variants"] = {"rounds": args.rounds, "order": "rotated each round", "results": rot,
                           "telemetry_per_round": clocks,
                           "telemetry_note": "sampled after each round, with the GPU idle (its clocks may "
                                             "read low); device.telemetry_under_load is the clock at work"}
        for v in variants:
            if v != ("owner", args.batch):
                del setups[v]
    del vol
    torch.cuda.empty_cache()

    if not args.no_cells:
        out["cells"] = config_cells(R, scenes, host_room, args)
    if not args.no_microbench:
        log("microbenchmarks")
        mb = out["microbench"] = microbench(torch, tsdf, stream)
        # the path against the measured ceilings: copy bandwidth, and the
        # atomic rates of the matching pattern
        t_upd = ktimes["k_update_owner"]["total_ms"] * 1e-3 / ktimes["k_update_owner"]["launches"]
        lds_per_clk = 2.0 * vox / launches_per_step / t_upd / 2.4e9 / 256    # two 64-bit LDS adds per voxel update
        ar = {
            "path_compulsory_frac_of_copy": round(out["path_roofline"]["achieved"] / mb["copy_GBps"], 5)
            if "path_roofline" in out else None,
            "k_update_owner": {"lds_u64_adds_per_clk_per_cu": round(lds_per_clk, 3),
                               "peak_random": mb["lds_add_u64_random_per_clk_per_cu"],
                               "peak_distinct": mb["lds_add_u64_distinct_per_clk_per_cu"],
                               "frac_of_random": round(lds_per_clk / mb["lds_add_u64_random_per_clk_per_cu"], 4),
                               "adds": "2 per voxel update (signed distance | count, colour), integer 64-bit"},
            "effective_bytes_40V": {"bytes_per_step": 40 * vox,
                                    "GBps": round(40 * vox * args.steps / wall / 1e9, 1),
                                    "note": "40 bytes per voxel update, as a per-visit read-modify-write would move: "
                                            "an effective figure, not traffic"},
        }
        if not args.no_variants and "rays_batch1" in out["variants"]["results"]:
            t_rays = out["variants"]["results"]["rays_batch1"]["step_ms"]["median"] * 1e-3
            g = 5.0 * vox / t_rays / 1e9
            # neighbouring rays add to neighbouring voxels, so the pattern lies
            # between the random rate and the coalesced one; the roof is the latter
            ar["rays_batch1"] = {"f32_atomics_Gops": round(g, 2),
                                 "peak_coalesced_Gops": mb["atomic_add_f32_coalesced_Gops"],
                                 "random_Gops": mb["atomic_add_f32_random_Gops"],
                                 "frac": round(g / mb["atomic_add_f32_coalesced_Gops"], 4),
                                 "atomics": "5 f32 adds per voxel update; step time includes allocate"}
        out["atomic_roofline"] = ar
    if args.sweep:
        log("sweep cells")
        out["sweep"] = sweep(R, scenes, args)
    out["device"]["telemetry_end"] = telemetry()
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_frames} frames")
        out["cpu_baseline"] = cpu_baseline(wl, host_room, args.cpu_frames)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
