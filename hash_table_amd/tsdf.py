"""ctypes binding of libtsdf_hip.so (include/tsdf.h, include/tsdf_microbench.h).

Argument marshalling only: every step of the integrate path runs in the HIP
kernels of the library.  The functions keep the C names; a status other than
TSDF_OK raises TsdfError.  PyTorch supplies device memory and streams
(``stream`` is an integer hipStream_t, e.g. ``torch.cuda.current_stream().cuda_stream``).

There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libtsdf_hip.so")

TSDF_OK, TSDF_EINVAL, TSDF_EALIGN, TSDF_EHIP, TSDF_ESMALL, TSDF_ELIMIT = 0, -1, -2, -3, -4, -5
TSDF_NOALLOC_SCRATCH_BYTES = 64 << 20
TSDF_UPDATE_OWNER, TSDF_UPDATE_RAYS = 0, 1
UPDATE_MODES = {"owner": TSDF_UPDATE_OWNER, "rays": TSDF_UPDATE_RAYS}
TSDF_OCCLUSION_RAY, TSDF_OCCLUSION_REPROJECT = 0, 1
OCCLUSION_MODES = {"ray": TSDF_OCCLUSION_RAY, "reproject": TSDF_OCCLUSION_REPROJECT}
TSDF_PROBE_BINS = 32
TSDF_MAX_BATCH = 128
TSDF_MAX_FRAME_SIDE = 65535
TSDF_MAX_POOL_BLOCKS = 1 << 30
TSDF_MAX_TABLE_ENTRIES = 1 << 31
BLOCK_VOXELS = 512
MB_COALESCED, MB_RANDOM, MB_SAME_WAVE, MB_BLOCK_ROW, MB_COUNTERS = 0, 1, 2, 3, 4
MB_LDS_U32, MB_LDS_F32, MB_LDS_U64 = 0, 1, 2
MB_LDS_DISTINCT, MB_LDS_RANDOM, MB_LDS_SAME, MB_LDS_GROUPS = 0, 1, 2, 3

# every symbol the headers declare
EXPORTS = [
    "tsdf_table_entries_for", "tsdf_counters_bytes", "tsdf_scratch_bytes", "tsdf_create", "tsdf_reset", "tsdf_allocate",
    "tsdf_update", "tsdf_integrate", "tsdf_integrate_batch", "tsdf_integrate_batch_noalloc", "tsdf_allocate_batch",
    "tsdf_update_batch",
    "tsdf_export_blocks", "tsdf_extract_mesh", "tsdf_get_stats", "tsdf_set_kernel_timing", "tsdf_kernel_times", "tsdf_destroy",
    "tsdf_status_str", "tsdf_mb_copy", "tsdf_mb_atomic_add_f32", "tsdf_mb_cas_u64", "tsdf_mb_lds_atomic",
]


class TsdfError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {_status_name(status)} ({status})")


class tsdf_config(ctypes.Structure):
    _fields_ = [("voxel_size", ctypes.c_float), ("trunc", ctypes.c_float),
                ("pool_capacity", ctypes.c_int64), ("table_entries", ctypes.c_int64),
                ("update_mode", ctypes.c_int32), ("max_batch_pixels", ctypes.c_int64),
                ("probe_limit", ctypes.c_int32), ("occlusion", ctypes.c_int32)]


class tsdf_buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("table", "tsdf", "weight", "r", "g", "b", "counters", "scratch")]


class tsdf_frame(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_void_p), ("rgb", ctypes.c_void_p),
                ("width", ctypes.c_int32), ("height", ctypes.c_int32),
                ("fx", ctypes.c_float), ("fy", ctypes.c_float), ("cx", ctypes.c_float), ("cy", ctypes.c_float),
                ("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3)]


class tsdf_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "pool_used", "pool_overflow", "table_full", "update_misses", "out_of_range", "near_skipped",
        "points_valid", "voxel_updates", "walk_guard", "probe_max", "fallback_blocks", "probe_exhausted")] + [
        ("probe_hist_alloc", ctypes.c_uint64 * TSDF_PROBE_BINS),
        ("probe_hist_update", ctypes.c_uint64 * TSDF_PROBE_BINS)]


class tsdf_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the HIP library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m hash_table_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "tsdf_table_entries_for": (I64, [I64]),
        "tsdf_counters_bytes": (SZ, []),
        "tsdf_scratch_bytes": (SZ, [ctypes.POINTER(tsdf_config)]),
        "tsdf_create": (I32, [ctypes.POINTER(tsdf_config), ctypes.POINTER(tsdf_buffers), P, ctypes.POINTER(P)]),
        "tsdf_reset": (I32, [P, P]),
        "tsdf_allocate": (I32, [P, ctypes.POINTER(tsdf_frame), P]),
        "tsdf_update": (I32, [P, ctypes.POINTER(tsdf_frame), P]),
        "tsdf_integrate": (I32, [P, ctypes.POINTER(tsdf_frame), P]),
        "tsdf_integrate_batch": (I32, [P, ctypes.POINTER(tsdf_frame), I32, P]),
        "tsdf_integrate_batch_noalloc": (I32, [P, ctypes.POINTER(tsdf_frame), I32, P]),
        "tsdf_allocate_batch": (I32, [P, ctypes.POINTER(tsdf_frame), I32, P]),
        "tsdf_update_batch": (I32, [P, ctypes.POINTER(tsdf_frame), I32, P]),
        "tsdf_export_blocks": (I32, [P, P, P, P, P, P, P, I64, ctypes.POINTER(I64), P]),
        "tsdf_extract_mesh": (I32, [P, P, P, I64, ctypes.POINTER(I64), P]),
        "tsdf_get_stats": (I32, [P, ctypes.POINTER(tsdf_stats), P]),
        "tsdf_set_kernel_timing": (I32, [P, I32]),
        "tsdf_kernel_times": (I32, [P, ctypes.POINTER(tsdf_kernel_time), I32, ctypes.POINTER(I32)]),
        "tsdf_destroy": (None, [P]),
        "tsdf_status_str": (ctypes.c_char_p, [I32]),
        "tsdf_mb_copy": (I32, [P, P, SZ, P]),
        "tsdf_mb_atomic_add_f32": (I32, [P, SZ, SZ, ctypes.c_int, ctypes.c_uint32, P]),
        "tsdf_mb_cas_u64": (I32, [P, SZ, SZ, ctypes.c_uint32, P]),
        "tsdf_mb_lds_atomic": (I32, [ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, P, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load().tsdf_status_str(status).decode()
    except Exception:
        return str(status)


def _check(status: int, call: str) -> None:
    if status != TSDF_OK:
        raise TsdfError(status, call)


# ---------------------------------------------------------------------------
# C entry points, same names
# ---------------------------------------------------------------------------
def tsdf_table_entries_for(pool_capacity: int) -> int:
    return int(load().tsdf_table_entries_for(pool_capacity))


def tsdf_counters_bytes() -> int:
    return int(load().tsdf_counters_bytes())


def tsdf_scratch_bytes(config: tsdf_config) -> int:
    return int(load().tsdf_scratch_bytes(ctypes.byref(config)))


def tsdf_status_str(status: int) -> str:
    return load().tsdf_status_str(status).decode()


def tsdf_create(config: tsdf_config, buffers: tsdf_buffers, stream: int = 0) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().tsdf_create(ctypes.byref(config), ctypes.byref(buffers), ctypes.c_void_p(stream),
                              ctypes.byref(h)), "tsdf_create")
    return h


def tsdf_reset(volume, stream: int = 0) -> None:
    _check(load().tsdf_reset(volume, ctypes.c_void_p(stream)), "tsdf_reset")


def tsdf_allocate(volume, frame: tsdf_frame, stream: int = 0) -> None:
    _check(load().tsdf_allocate(volume, ctypes.byref(frame), ctypes.c_void_p(stream)), "tsdf_allocate")


def tsdf_update(volume, frame: tsdf_frame, stream: int = 0) -> None:
    _check(load().tsdf_update(volume, ctypes.byref(frame), ctypes.c_void_p(stream)), "tsdf_update")


def tsdf_integrate(volume, frame: tsdf_frame, stream: int = 0) -> None:
    _check(load().tsdf_integrate(volume, ctypes.byref(frame), ctypes.c_void_p(stream)), "tsdf_integrate")


def frame_array(frames) -> ctypes.Array:
    """A ctypes array of tsdf_frame from a sequence (or pass an array through)."""
    if isinstance(frames, ctypes.Array):
        return frames
    return (tsdf_frame * max(len(frames), 1))(*frames)


def tsdf_integrate_batch(volume, frames, stream: int = 0, n: Optional[int] = None) -> None:
    arr = frame_array(frames)
    _check(load().tsdf_integrate_batch(volume, arr, len(frames) if n is None else n, ctypes.c_void_p(stream)),
           "tsdf_integrate_batch")


def tsdf_integrate_batch_noalloc(volume, frames, stream: int = 0, n: Optional[int] = None) -> None:
    arr = frame_array(frames)
    _check(load().tsdf_integrate_batch_noalloc(volume, arr, len(frames) if n is None else n,
                                               ctypes.c_void_p(stream)), "tsdf_integrate_batch_noalloc")


def tsdf_allocate_batch(volume, frames, stream: int = 0, n: Optional[int] = None) -> None:
    arr = frame_array(frames)
    _check(load().tsdf_allocate_batch(volume, arr, len(frames) if n is None else n, ctypes.c_void_p(stream)),
           "tsdf_allocate_batch")


def tsdf_update_batch(volume, frames, stream: int = 0, n: Optional[int] = None) -> None:
    arr = frame_array(frames)
    _check(load().tsdf_update_batch(volume, arr, len(frames) if n is None else n, ctypes.c_void_p(stream)),
           "tsdf_update_batch")


def tsdf_export_blocks(volume, coords: int, tsdf: int, weight: int, r: int, g: int, b: int,
                       max_blocks: int, stream: int = 0) -> int:
    n = ctypes.c_int64(0)
    st = load().tsdf_export_blocks(volume, *(ctypes.c_void_p(p) for p in (coords, tsdf, weight, r, g, b)),
                                   max_blocks, ctypes.byref(n), ctypes.c_void_p(stream))
    if st == TSDF_ESMALL:
        raise TsdfError(st, f"tsdf_export_blocks ({n.value} blocks > {max_blocks})")
    _check(st, "tsdf_export_blocks")
    return int(n.value)


def tsdf_extract_mesh(volume, positions: int, keys: int, max_triangles: int, stream: int = 0) -> int:
    """Returns the number of triangles (raises TsdfError(TSDF_ESMALL) if more
    than max_triangles; the count is then in the error's `n_triangles`)."""
    n = ctypes.c_int64(0)
    st = load().tsdf_extract_mesh(volume, ctypes.c_void_p(positions), ctypes.c_void_p(keys), max_triangles,
                                  ctypes.byref(n), ctypes.c_void_p(stream))
    if st == TSDF_ESMALL:
        e = TsdfError(st, f"tsdf_extract_mesh ({n.value} triangles > {max_triangles})")
        e.n_triangles = int(n.value)
        raise e
    _check(st, "tsdf_extract_mesh")
    return int(n.value)


def tsdf_get_stats(volume, stream: int = 0) -> Dict[str, object]:
    s = tsdf_stats()
    _check(load().tsdf_get_stats(volume, ctypes.byref(s), ctypes.c_void_p(stream)), "tsdf_get_stats")
    out: Dict[str, object] = {n: int(getattr(s, n)) for n, _ in tsdf_stats._fields_[:12]}
    out["probe_hist_alloc"] = np.array(s.probe_hist_alloc[:], np.int64)
    out["probe_hist_update"] = np.array(s.probe_hist_update[:], np.int64)
    return out


def tsdf_set_kernel_timing(volume, enable: bool) -> None:
    _check(load().tsdf_set_kernel_timing(volume, 1 if enable else 0), "tsdf_set_kernel_timing")


def tsdf_kernel_times(volume) -> Dict[str, Dict[str, float]]:
    """{kernel name: {"launches": n, "total_ms": ms}} since timing was enabled
    or last read (waits for the recorded events)."""
    out = (tsdf_kernel_time * 16)()
    n = ctypes.c_int32(0)
    _check(load().tsdf_kernel_times(volume, out, 16, ctypes.byref(n)), "tsdf_kernel_times")
    return {out[i].name.decode(): {"launches": int(out[i].launches), "total_ms": float(out[i].total_ms)}
            for i in range(n.value)}


def tsdf_destroy(volume) -> None:
    if volume:
        load().tsdf_destroy(volume)


def tsdf_mb_copy(src: int, dst: int, nbytes: int, stream: int = 0) -> None:
    _check(load().tsdf_mb_copy(src, dst, nbytes, ctypes.c_void_p(stream)), "tsdf_mb_copy")


def tsdf_mb_atomic_add_f32(buf: int, n: int, n_ops: int, pattern: int, seed: int = 1, stream: int = 0) -> None:
    _check(load().tsdf_mb_atomic_add_f32(buf, n, n_ops, pattern, seed, ctypes.c_void_p(stream)),
           "tsdf_mb_atomic_add_f32")


def tsdf_mb_cas_u64(buf: int, n: int, n_ops: int, seed: int = 1, stream: int = 0) -> None:
    _check(load().tsdf_mb_cas_u64(buf, n, n_ops, seed, ctypes.c_void_p(stream)), "tsdf_mb_cas_u64")


def tsdf_mb_lds_atomic(type_: int, pattern: int, n_workgroups: int, iters: int, sink: int, stream: int = 0) -> None:
    _check(load().tsdf_mb_lds_atomic(type_, pattern, n_workgroups, iters, ctypes.c_void_p(sink),
                                     ctypes.c_void_p(stream)), "tsdf_mb_lds_atomic")


# ---------------------------------------------------------------------------
# torch-backed convenience wrappers (memory and streams only)
# ---------------------------------------------------------------------------
def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class DeviceFrame:
    """A frame uploaded to device memory, with its tsdf_frame descriptor."""

    def __init__(self, frame, device="cuda"):
        import torch
        self.depth = torch.from_numpy(np.ascontiguousarray(frame.depth, np.float32)).to(device)
        self.rgb = torch.from_numpy(np.ascontiguousarray(frame.rgb, np.uint8)).to(device)
        H, W = self.depth.shape
        f = tsdf_frame()
        f.depth = self.depth.data_ptr() if self.depth.numel() else None
        f.rgb = self.rgb.data_ptr() if self.rgb.numel() else None
        f.width, f.height = W, H
        f.fx, f.fy, f.cx, f.cy = frame.fx, frame.fy, frame.cx, frame.cy
        R = np.ascontiguousarray(frame.R, np.float32).reshape(9)
        t = np.ascontiguousarray(frame.t, np.float32).reshape(3)
        f.R = (ctypes.c_float * 9)(*R.tolist())
        f.t = (ctypes.c_float * 3)(*t.tolist())
        self.desc = f
        self.valid_hint = None


class Volume:
    """A TSDF volume whose table, pool, counters and scratch are torch CUDA
    tensors.  update_mode: "owner" (default) or "rays"."""

    def __init__(self, voxel_size: float, trunc: float, pool_capacity: int, table_entries: int = 0,
                 update_mode: str = "owner", max_batch_pixels: int = 0, device="cuda", stream=None,
                 probe_limit: int = 0, occlusion: str = "ray"):
        import torch
        entries = table_entries or tsdf_table_entries_for(pool_capacity)
        if entries <= 0:
            raise TsdfError(TSDF_EINVAL, "tsdf_table_entries_for")
        self.voxel_size, self.trunc = voxel_size, trunc
        self.pool_capacity, self.table_entries = int(pool_capacity), int(entries)
        self.update_mode = update_mode
        self.device = device
        self._cfg = tsdf_config(voxel_size, trunc, int(pool_capacity), int(table_entries), UPDATE_MODES[update_mode],
                                int(max_batch_pixels), int(probe_limit), OCCLUSION_MODES[occlusion])
        n = int(pool_capacity) * BLOCK_VOXELS
        self.table = torch.empty(int(entries) * 2, dtype=torch.int64, device=device)
        self.pool = {k: torch.empty(n, dtype=torch.float32, device=device) for k in ("tsdf", "weight", "r", "g", "b")}
        self.counters = torch.empty((tsdf_counters_bytes() + 7) // 8, dtype=torch.int64, device=device)
        scratch = tsdf_scratch_bytes(self._cfg)
        self.scratch = torch.empty((scratch + 7) // 8, dtype=torch.int64, device=device) if scratch else None
        self._buf = tsdf_buffers(self.table.data_ptr(), *(self.pool[k].data_ptr() for k in
                                 ("tsdf", "weight", "r", "g", "b")), self.counters.data_ptr(),
                                 self.scratch.data_ptr() if scratch else None)
        self.handle = tsdf_create(self._cfg, self._buf, _stream_handle(stream))

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                tsdf_destroy(h)
            except TypeError:               # interpreter shutdown: module globals already gone
                pass
            self.handle = None

    def reset(self, stream=None):
        tsdf_reset(self.handle, _stream_handle(stream))

    def allocate(self, frame: DeviceFrame, stream=None):
        tsdf_allocate(self.handle, frame.desc, _stream_handle(stream))

    def update(self, frame: DeviceFrame, stream=None):
        tsdf_update(self.handle, frame.desc, _stream_handle(stream))

    def integrate(self, frame: DeviceFrame, stream=None):
        tsdf_integrate(self.handle, frame.desc, _stream_handle(stream))

    def integrate_batch(self, frames, stream=None):
        tsdf_integrate_batch(self.handle, [f.desc for f in frames], _stream_handle(stream))

    def stats(self, stream=None) -> Dict[str, object]:
        return tsdf_get_stats(self.handle, _stream_handle(stream))

    def set_kernel_timing(self, enable: bool = True) -> None:
        tsdf_set_kernel_timing(self.handle, enable)

    def kernel_times(self) -> Dict[str, Dict[str, float]]:
        return tsdf_kernel_times(self.handle)

    def extract_mesh(self, stream=None, with_keys=True):
        """Marching tetrahedra on the device: host arrays positions
        (n, 3, 3) float32 metres and keys (n, 3, 4) int32 (vertex names).
        A count-only call sizes the output first."""
        import torch
        sh = _stream_handle(stream)
        try:
            n = tsdf_extract_mesh(self.handle, 0, 0, 0, sh)
        except TsdfError as e:
            if e.status != TSDF_ESMALL:
                raise
            n = e.n_triangles
        pos = torch.empty((max(n, 1), 9), dtype=torch.float32, device=self.device)
        key = torch.empty((max(n, 1), 12), dtype=torch.int32, device=self.device) if with_keys else None
        got = tsdf_extract_mesh(self.handle, pos.data_ptr(), key.data_ptr() if with_keys else 0, n, sh)
        assert got == n, (got, n)
        out_pos = pos[:n].cpu().numpy().reshape(n, 3, 3)
        out_key = key[:n].cpu().numpy().reshape(n, 3, 4) if with_keys else None
        return out_pos, out_key

    def export(self, stream=None, arrays=("tsdf", "weight", "r", "g", "b")):
        """All pool blocks as host numpy arrays: coords (n, 3) int32 and
        {name: (n, 512) float32}, in pool-index order."""
        import torch
        n = int(self.stats(stream)["pool_used"])
        coords = torch.empty((max(n, 1), 3), dtype=torch.int32, device=self.device)
        outs = {k: torch.empty((max(n, 1), BLOCK_VOXELS), dtype=torch.float32, device=self.device) for k in arrays}
        ptr = {k: (outs[k].data_ptr() if k in outs else 0) for k in ("tsdf", "weight", "r", "g", "b")}
        got = tsdf_export_blocks(self.handle, coords.data_ptr(), ptr["tsdf"], ptr["weight"], ptr["r"], ptr["g"],
                                 ptr["b"], max(n, 1), _stream_handle(stream))
        assert got == n, (got, n)
        return coords[:n].cpu().numpy(), {k: v[:n].cpu().numpy() for k, v in outs.items()}
