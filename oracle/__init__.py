"""Reference ("oracle") integrator and surface extraction for hash-blocked
TSDF fusion.

TEST INFRASTRUCTURE ONLY.  A plain, single-threaded C++ implementation
(``tsdf_oracle.cpp``, a ``std::map`` keyed by block coordinate; and
``mesh_oracle.cpp``, marching tetrahedra over the fused volume) that the
tests, the smoke check and the benchmark's CPU-baseline leg use to check and
time the HIP library.  The HIP library and its Python binding never import,
load or call anything here, and share no code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Iterable

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "tsdf_oracle.cpp")
LIBRARY = os.path.join(HERE, "libtsdf_oracle.so")
MESH_SOURCE = os.path.join(HERE, "mesh_oracle.cpp")          # marching tetrahedra (surface extraction)
MESH_LIBRARY = os.path.join(HERE, "libmesh_oracle.so")

# Strict IEEE single precision: no contraction into FMA, no fast-math, SSE
# arithmetic (x86-64 default) so no excess precision.
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-mfpmath=sse", "-fno-finite-math-only"]

TRACK_TOUCHED = 1
REPROJECT = 4          # the reprojection reading of the occlusion test (C8)


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags: Iterable[str] = ()) -> str:
    """Compile the oracle (or a copy of its source) into a shared library;
    with no arguments also the extraction oracle."""
    tmp = output + f".tmp{os.getpid()}"
    cmd = ["g++", *CXXFLAGS, *extra_flags, "-o", tmp, source]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    if source == SOURCE and output == LIBRARY:
        build(MESH_SOURCE, MESH_LIBRARY, extra_flags)
    return output


class _FrameStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "pixels", "points_valid", "near_skipped", "out_of_range", "cells_visited",
        "voxel_updates", "blocks_touched", "blocks_new", "voxels_touched",
        "update_misses", "pool_overflow_new")]


class _CallStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "frames", "blocks_touched", "blocks_new", "voxels_fresh", "voxels_old")]


class _Totals(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "blocks", "pool_overflow", "update_misses", "points_valid", "near_skipped",
        "out_of_range", "voxel_updates", "frames")]


_LIBS: Dict[str, ctypes.CDLL] = {}


def load(path: str = LIBRARY) -> ctypes.CDLL:
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        if path != LIBRARY:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_create.restype = P
    lib.oracle_create.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_int64, ctypes.c_int32]
    lib.oracle_destroy.argtypes = [P]
    lib.oracle_begin_call.argtypes = [P]
    lib.oracle_get_call_stats.argtypes = [P, ctypes.POINTER(_CallStats)]
    lib.oracle_integrate.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                     P, P, ctypes.POINTER(_FrameStats)]
    lib.oracle_get_totals.argtypes = [P, ctypes.POINTER(_Totals)]
    lib.oracle_block_count.restype = ctypes.c_int64
    lib.oracle_block_count.argtypes = [P]
    lib.oracle_block_coords.argtypes = [P, P]
    lib.oracle_block_sums.restype = ctypes.c_int64
    lib.oracle_block_sums.argtypes = [P, P, ctypes.c_int64, P, P, P, P, P]
    _LIBS[path] = lib
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def load_mesh(path: str = MESH_LIBRARY) -> ctypes.CDLL:
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        if path != MESH_LIBRARY:
            raise FileNotFoundError(path)
        build(MESH_SOURCE, MESH_LIBRARY)
    lib = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_mesh.restype = P
    lib.oracle_mesh.argtypes = [P, P, P, I64, ctypes.c_double]
    lib.oracle_mesh_vertex_count.restype = I64
    lib.oracle_mesh_vertex_count.argtypes = [P]
    lib.oracle_mesh_triangle_count.restype = I64
    lib.oracle_mesh_triangle_count.argtypes = [P]
    lib.oracle_mesh_vertices.argtypes = [P, P, P]
    lib.oracle_mesh_triangles.argtypes = [P, P]
    lib.oracle_mesh_destroy.argtypes = [P]
    _LIBS[path] = lib
    return lib


class Mesh:
    """The extraction oracle's surface: keys (nv, 4) int32 -- the edge's lower
    lattice point (voxel coordinates) and direction d = dx | dy << 1 | dz << 2
    --, positions (nv, 3) float64 in metres, triangles (nt, 3) indices into
    the vertex arrays, each oriented with its normal from inside to outside."""

    def __init__(self, keys, pos, tris):
        self.keys, self.pos, self.tris = keys, pos, tris


def extract_mesh(coords: np.ndarray, tsdf: np.ndarray, weight: np.ndarray, voxel_size: float,
                 library: str = MESH_LIBRARY) -> Mesh:
    """Marching tetrahedra over blocks (coords (n, 3); tsdf and weight sums
    (n, 512)): the extraction oracle of mesh_oracle.cpp."""
    lib = load_mesh(library)
    c = np.ascontiguousarray(coords, np.int32).reshape(-1, 3)
    t = np.ascontiguousarray(tsdf, np.float64).reshape(-1, 512)
    w = np.ascontiguousarray(weight, np.float64).reshape(-1, 512)
    assert t.shape[0] == w.shape[0] == c.shape[0]
    h = lib.oracle_mesh(_ptr(c), _ptr(t), _ptr(w), c.shape[0], float(voxel_size))
    try:
        nv, nt = int(lib.oracle_mesh_vertex_count(h)), int(lib.oracle_mesh_triangle_count(h))
        keys = np.empty((nv, 4), np.int32)
        pos = np.empty((nv, 3), np.float64)
        tris = np.empty((nt, 3), np.int64)
        if nv:
            lib.oracle_mesh_vertices(h, _ptr(keys), _ptr(pos))
        if nt:
            lib.oracle_mesh_triangles(h, _ptr(tris))
    finally:
        lib.oracle_mesh_destroy(h)
    return Mesh(keys, pos, tris)


class Oracle:
    """One volume integrated by the reference implementation.

    pool_capacity bounds the number of blocks; keys beyond it are refused and
    counted.  track_touched enables the distinct-voxel counts (U per frame,
    voxels_fresh / voxels_old per call); reproject selects the reprojection
    reading of the occlusion test (C8)."""

    def __init__(self, voxel_size: float, trunc: float, pool_capacity: int,
                 track_touched: bool = False, library: str = LIBRARY, reproject: bool = False):
        self._lib = load(library)
        flags = (TRACK_TOUCHED if track_touched else 0) | (REPROJECT if reproject else 0)
        self._h = self._lib.oracle_create(voxel_size, trunc, int(pool_capacity), flags)
        if not self._h:
            raise ValueError("invalid oracle parameters")
        self.frame_stats = []

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.oracle_destroy(h)
            self._h = None

    def integrate(self, frame) -> dict:
        depth = np.ascontiguousarray(frame.depth, np.float32)
        rgb = np.ascontiguousarray(frame.rgb, np.uint8)
        H, W = depth.shape
        assert rgb.shape == (H, W, 3)
        R = np.ascontiguousarray(frame.R, np.float32).reshape(9)
        t = np.ascontiguousarray(frame.t, np.float32).reshape(3)
        st = _FrameStats()
        rc = self._lib.oracle_integrate(self._h, _ptr(depth), _ptr(rgb), W, H,
                                        frame.fx, frame.fy, frame.cx, frame.cy,
                                        _ptr(R), _ptr(t), ctypes.byref(st))
        if rc != 0:
            raise RuntimeError(f"oracle_integrate failed ({rc})")
        d = {n: int(getattr(st, n)) for n, _ in _FrameStats._fields_}
        self.frame_stats.append(d)
        return d

    def begin_call(self) -> None:
        """Count the frames integrated from here on as one call (batch)."""
        self._lib.oracle_begin_call(self._h)

    def call_stats(self) -> dict:
        """Counts of the current call: frames, distinct blocks touched (B_call),
        blocks created, distinct voxels touched in blocks the call created
        (voxels_fresh) and in older blocks (voxels_old)."""
        c = _CallStats()
        self._lib.oracle_get_call_stats(self._h, ctypes.byref(c))
        return {n: int(getattr(c, n)) for n, _ in _CallStats._fields_}

    def totals(self) -> dict:
        t = _Totals()
        self._lib.oracle_get_totals(self._h, ctypes.byref(t))
        return {n: int(getattr(t, n)) for n, _ in _Totals._fields_}

    def block_count(self) -> int:
        return int(self._lib.oracle_block_count(self._h))

    def block_coords(self) -> np.ndarray:
        n = self.block_count()
        out = np.empty((n, 3), np.int32)
        if n:
            self._lib.oracle_block_coords(self._h, _ptr(out))
        return out

    def block_sums(self, coords: np.ndarray) -> Dict[str, np.ndarray]:
        c = np.ascontiguousarray(coords, np.int32).reshape(-1, 3)
        n = c.shape[0]
        out = {k: np.empty((n, 512), np.float64) for k in ("tsdf", "weight", "r", "g", "b")}
        if n:
            self._lib.oracle_block_sums(self._h, _ptr(c), n, _ptr(out["tsdf"]), _ptr(out["weight"]),
                                        _ptr(out["r"]), _ptr(out["g"]), _ptr(out["b"]))
        return out
