"""Seeded synthetic depth + colour workloads for hash-blocked TSDF integration.

This module is the only thing the HIP path and the oracle share: it renders
depth frames (camera-z of the first ray hit, metres, float32) and uint8 RGB
frames of analytic scenes, with the camera-to-world pose of every frame.  It
holds scene geometry and ray casting only, none of the fusion arithmetic.

Scenes follow the workloads that "What Irregularity Costs: CUDA C++, Rust, and
Triton on a Hash-Blocked GPU Workload" measures on (an analytic sphere, a plane,
room-scale depth trajectories, a load-factor sweep and a contention cell);
its real-depth trajectories are not available, so the room scenes stand in
for their shape.

Conventions (OpenCV pinhole):
  * pixel (u, v) is column u, row v; the ray through it has camera-frame
    direction ((u - cx) / fx, (v - cy) / fy, 1), so a ray parameter equals
    camera z;
  * camera axes: x right, y down, z forward; at the identity pose they match
    the world axes, so the world is y-down (floors have the largest y);
  * pose = (R, t) with p_world = R @ p_cam + t, R row-major float32.

Everything is generated in float64 from ``numpy.random.default_rng(seed)``
and cast to float32 / uint8 at the end.
"""
from __future__ import annotations

import hashlib
import math
import re
from dataclasses import dataclass, field
from typing import Callable, Iterator, List, Optional

import numpy as np

__all__ = [
    "Frame", "Workload", "workload", "plane_frame", "random_frame",
    "frame_digest", "next_pow2", "WORKLOADS", "room_cell", "cell_name", "SWEEP_CELLS",
    "load_factor_cell", "LOAD_FACTORS", "BENCH_CALLS",
]


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------
@dataclass
class Frame:
    depth: np.ndarray          # (H, W) float32, metres of camera z, 0 = invalid
    rgb: np.ndarray            # (H, W, 3) uint8
    fx: float
    fy: float
    cx: float
    cy: float
    R: np.ndarray              # (3, 3) float32, camera -> world rotation
    t: np.ndarray              # (3,) float32, camera centre in world

    @property
    def width(self) -> int:
        return int(self.depth.shape[1])

    @property
    def height(self) -> int:
        return int(self.depth.shape[0])


@dataclass
class Workload:
    name: str
    width: int
    height: int
    voxel_size: float
    trunc: float
    pool_capacity: int
    table_entries: int
    n_frames: int
    make_frame: Callable[[int], Frame] = field(repr=False)
    description: str = ""

    def frame(self, i: int) -> Frame:
        if not 0 <= i < self.n_frames:
            raise IndexError(i)
        return self.make_frame(i)

    def frames(self, start: int = 0, stop: Optional[int] = None) -> Iterator[Frame]:
        stop = self.n_frames if stop is None else min(stop, self.n_frames)
        for i in range(start, stop):
            yield self.make_frame(i)


def next_pow2(n: int) -> int:
    """Smallest power of two >= n (n >= 1)."""
    n = int(n)
    if n < 1:
        raise ValueError(n)
    return 1 << (n - 1).bit_length()


def frame_digest(frames: List[Frame]) -> str:
    """SHA-256 over every array and camera parameter of a frame list."""
    h = hashlib.sha256()
    for f in frames:
        h.update(np.ascontiguousarray(f.depth).tobytes())
        h.update(np.ascontiguousarray(f.rgb).tobytes())
        h.update(np.asarray([f.fx, f.fy, f.cx, f.cy], np.float32).tobytes())
        h.update(np.ascontiguousarray(f.R, np.float32).tobytes())
        h.update(np.ascontiguousarray(f.t, np.float32).tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------
# camera helpers
# --------------------------------------------------------------------------
_DOWN = np.array([0.0, 1.0, 0.0])


def _look_rotation(forward: np.ndarray) -> np.ndarray:
    """Camera->world rotation whose z axis is `forward` and whose y axis points
    as far down (+y) as possible."""
    f = forward / np.linalg.norm(forward)
    r = np.cross(_DOWN, f)
    r /= np.linalg.norm(r)
    d = np.cross(f, r)
    return np.stack([r, d, f], axis=1)


def _yaw_pitch_rotation(yaw: float, pitch: float) -> np.ndarray:
    f = np.array([math.cos(pitch) * math.sin(yaw), -math.sin(pitch),
                  math.cos(pitch) * math.cos(yaw)])
    return _look_rotation(f)


def _ray_dirs(W, H, fx, fy, cx, cy, R):
    """World-space ray directions (H*W, 3) whose camera-z component is 1."""
    u = (np.arange(W, dtype=np.float64) - cx) / fx
    v = (np.arange(H, dtype=np.float64) - cy) / fy
    dc = np.empty((H, W, 3))
    dc[..., 0] = u[None, :]
    dc[..., 1] = v[:, None]
    dc[..., 2] = 1.0
    return dc.reshape(-1, 3) @ R.T


def _u8(c: np.ndarray) -> np.ndarray:
    return np.clip(np.floor(255.0 * np.asarray(c, np.float64) + 0.5), 0, 255).astype(np.uint8)


# --------------------------------------------------------------------------
# ray casting (float64); every cast returns (t, object id) per ray, t = inf on miss
# --------------------------------------------------------------------------
_BOX_EDGES = [(a, b) for a in range(8) for b in range(8)
              if a < b and bin(a ^ b).count("1") == 1]


def _screen_rect(corners_w, o, R, fx, fy, cx, cy, W, H, near=1e-3):
    """Pixel rectangle (u0, u1, v0, v1), half-open, that covers the projection
    of the part of a world-space box (8 corners, index bits = x/y/z max) in
    front of the plane z_cam = near; None if nothing of it is on screen."""
    pc = (corners_w - o) @ R            # rows: R^T (p - o)
    z = pc[:, 2]
    pts = [pc[z > near]]
    if np.any(z <= near):
        if np.all(z <= near):
            return None
        for a, b in _BOX_EDGES:         # edge / near-plane crossings
            if (z[a] > near) != (z[b] > near):
                s = (near - z[a]) / (z[b] - z[a])
                pts.append((pc[a] + s * (pc[b] - pc[a]))[None, :])
    p = np.concatenate(pts)
    zz = np.maximum(p[:, 2], near)
    u = fx * p[:, 0] / zz + cx
    v = fy * p[:, 1] / zz + cy
    u0 = max(int(math.floor(max(u.min(), -1e9))) - 1, 0)
    u1 = min(int(math.ceil(min(u.max(), 1e9))) + 2, W)
    v0 = max(int(math.floor(max(v.min(), -1e9))) - 1, 0)
    v1 = min(int(math.ceil(min(v.max(), 1e9))) + 2, H)
    if u0 >= u1 or v0 >= v1:
        return None
    return u0, u1, v0, v1


def _box_corners(bmin, bmax):
    return np.array([[x, y, z] for x in (bmin[0], bmax[0])
                     for y in (bmin[1], bmax[1]) for z in (bmin[2], bmax[2])])


def _hit_box(o, d, bmin, bmax):
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = 1.0 / d
        t1 = (bmin - o) * inv
        t2 = (bmax - o) * inv
        tn = np.nanmax(np.minimum(t1, t2), axis=1)
        tf = np.nanmin(np.maximum(t1, t2), axis=1)
    hit = (tn <= tf) & (tn > 1e-6)
    return np.where(hit, tn, np.inf)


def _hit_sphere(o, d, c, r):
    oc = o - c
    a = np.einsum("ij,ij->i", d, d)
    b = d @ oc
    cc = oc @ oc - r * r
    disc = b * b - a * cc
    with np.errstate(invalid="ignore"):
        t = (-b - np.sqrt(disc)) / a
    hit = (disc >= 0) & (t > 1e-6)
    return np.where(hit, t, np.inf)


def _cast_scene(o, R, fx, fy, cx, cy, W, H, boxes, spheres, room=None, planes=()):
    """First-hit ray cast.  boxes: list of (bmin, bmax); spheres: list of
    (centre, radius); room: (rmin, rmax) seen from inside, ids -1..-6 for its
    faces; planes: list of (axis, value) infinite planes, ids -(10+k).
    Returns (t, id) with id = index into boxes, then len(boxes)+index into
    spheres, negative for room faces and planes."""
    d = _ray_dirs(W, H, fx, fy, cx, cy, R)
    n = d.shape[0]
    t = np.full(n, np.inf)
    oid = np.full(n, -1000, np.int64)
    if room is not None:
        rmin, rmax = room
        with np.errstate(divide="ignore", invalid="ignore"):
            bound = np.where(d > 0, rmax, rmin)
            ti = (bound - o) / d
        ti = np.where(np.isfinite(ti) & (ti > 0), ti, np.inf)
        ax = np.argmin(ti, axis=1)
        t = ti[np.arange(n), ax]
        side = (d[np.arange(n), ax] > 0).astype(np.int64)
        oid = -(1 + 2 * ax + side)          # -1..-6
    for k, (axis, val) in enumerate(planes):
        with np.errstate(divide="ignore", invalid="ignore"):
            tp = (val - o[axis]) / d[:, axis]
        tp = np.where(np.isfinite(tp) & (tp > 0), tp, np.inf)
        closer = tp < t
        t = np.where(closer, tp, t)
        oid = np.where(closer, -(10 + k), oid)
    img_idx = np.arange(n).reshape(H, W)
    for k, (bmin, bmax) in enumerate(boxes):
        rect = _screen_rect(_box_corners(bmin, bmax), o, R, fx, fy, cx, cy, W, H)
        if rect is None:
            continue
        u0, u1, v0, v1 = rect
        idx = img_idx[v0:v1, u0:u1].ravel()
        tb = _hit_box(o, d[idx], np.asarray(bmin), np.asarray(bmax))
        closer = tb < t[idx]
        t[idx[closer]] = tb[closer]
        oid[idx[closer]] = k
    for k, (c, r) in enumerate(spheres):
        c = np.asarray(c, np.float64)
        rect = _screen_rect(_box_corners(c - r, c + r), o, R, fx, fy, cx, cy, W, H)
        if rect is None:
            continue
        u0, u1, v0, v1 = rect
        idx = img_idx[v0:v1, u0:u1].ravel()
        ts = _hit_sphere(o, d[idx], c, r)
        closer = ts < t[idx]
        t[idx[closer]] = ts[closer]
        oid[idx[closer]] = len(boxes) + k
    return t.reshape(H, W), oid.reshape(H, W), d.reshape(H, W, 3)


def _finish_depth(t, rng, sigma, zero_frac):
    depth = t.copy()
    depth[~np.isfinite(depth)] = 0.0
    if sigma > 0:
        depth = depth + rng.normal(0.0, sigma, depth.shape) * (depth > 0)
    if zero_frac > 0:
        depth[rng.random(depth.shape) < zero_frac] = 0.0
    depth[depth < 0] = 0.0
    return depth.astype(np.float32)


def _frame(depth, rgb, fx, fy, cx, cy, R, t):
    return Frame(depth=np.ascontiguousarray(depth, np.float32),
                 rgb=np.ascontiguousarray(rgb, np.uint8),
                 fx=float(np.float32(fx)), fy=float(np.float32(fy)),
                 cx=float(np.float32(cx)), cy=float(np.float32(cy)),
                 R=np.ascontiguousarray(R, np.float32),
                 t=np.ascontiguousarray(t, np.float32))


# --------------------------------------------------------------------------
# workload 1: fronto-parallel plane
# --------------------------------------------------------------------------
def plane_frame(seed=1, W=64, H=48, depth=1.0, fx=50.0, fy=50.0, cx=32.0, cy=24.0):
    """Constant-depth frame (a plane facing an identity-pose camera) with
    uniform random uint8 colour."""
    rng = np.random.default_rng(seed)
    rgb = rng.integers(0, 256, size=(H, W, 3), dtype=np.uint8)
    d = np.full((H, W), depth, np.float32)
    return _frame(d, rgb, fx, fy, cx, cy, np.eye(3), np.zeros(3))


def _plane_workload():
    f = plane_frame()
    return Workload("plane64x48", 64, 48, 0.01, 0.04, 4096, 8192, 1,
                    lambda i: plane_frame(),
                    "single 64x48 fronto-parallel plane at z = 1 m")


# --------------------------------------------------------------------------
# workload 2: sphere in front of a wall, camera on an arc
# --------------------------------------------------------------------------
def _smooth_colour(rng):
    freq = rng.uniform(0.5, 2.0, size=(3, 3)) * rng.choice([-1.0, 1.0], size=(3, 3))
    phase = rng.uniform(0.0, 2.0 * math.pi, size=3)

    def colour(p):                                # p (..., 3) world points
        return 0.5 + 0.5 * np.sin(2.0 * math.pi * (p @ freq.T) + phase)
    return colour


def _sphere_wall_workload(sigma=0.002, n_frames=10, W=320, H=240, seed=2):
    fx = fy = 300.0
    cx, cy = (W - 1) / 2.0, (H - 1) / 2.0
    centre = np.array([0.0, 0.0, 1.5])
    colour = _smooth_colour(np.random.default_rng([seed, 0]))

    def make(i):
        th = math.radians(15.0) * i / 9.0
        o = np.array([-1.5 * math.sin(th), 0.0, 1.5 - 1.5 * math.cos(th)])
        R = _look_rotation(centre - o)
        t, oid, d = _cast_scene(o, R, fx, fy, cx, cy, W, H, [], [(centre, 0.5)],
                                planes=[(2, 3.0)])
        p = o + t[..., None] * d
        p[~np.isfinite(t)] = 0.0
        rgb = _u8(colour(p))
        rng = np.random.default_rng([seed, 1, i])
        depth = _finish_depth(t, rng, sigma, 0.0)
        return _frame(depth, rgb, fx, fy, cx, cy, R, o)

    name = "spherewall320x240" + ("" if sigma > 0 else "_noisefree")
    return Workload(name, W, H, 0.01, 0.04, 65536, 131072, n_frames, make,
                    "sphere r=0.5 at (0,0,1.5) before a wall at z=3, 15 deg arc")


# --------------------------------------------------------------------------
# room scenes (workloads 3, 4, 5): smoothed random-walk camera among boxes
# --------------------------------------------------------------------------
def _random_walk(rng, n, lo, hi, y_lo, y_hi, step=0.015):
    """Smoothed random-walk trajectory: AR(1) velocity (about `step` m per
    frame) and yaw rate (under 1 deg per frame), pitch within +-10 deg.
    Returns (positions (n,3), yaw (n,), pitch (n,))."""
    pos = np.empty((n, 3))
    yaws = np.empty(n)
    pitches = np.empty(n)
    p = np.array([rng.uniform(lo * 0.3, hi * 0.3), rng.uniform(y_lo, y_hi),
                  rng.uniform(lo * 0.3, hi * 0.3)])
    heading = rng.uniform(0, 2 * math.pi)
    v = step * np.array([math.sin(heading), 0.0, math.cos(heading)])
    yaw = rng.uniform(0, 2 * math.pi)
    yaw_rate = 0.0
    pitch = 0.0
    lim = math.radians(10.0)
    for k in range(n):
        v = 0.9 * v + rng.normal(0.0, 0.3 * step, 3) * np.array([1.0, 0.2, 1.0])
        sp = np.linalg.norm(v)
        if sp > 2.0 * step:
            v *= 2.0 * step / sp
        p = p + v
        for a, (a_lo, a_hi) in enumerate(((lo, hi), (y_lo, y_hi), (lo, hi))):
            if p[a] < a_lo:
                p[a] = 2 * a_lo - p[a]
                v[a] = abs(v[a])
            elif p[a] > a_hi:
                p[a] = 2 * a_hi - p[a]
                v[a] = -abs(v[a])
        yaw_rate = 0.85 * yaw_rate + rng.normal(0.0, math.radians(0.25))
        yaw_rate = float(np.clip(yaw_rate, -math.radians(1.0), math.radians(1.0)))
        yaw += yaw_rate
        pitch = float(np.clip(0.95 * pitch + rng.normal(0.0, math.radians(0.4)), -lim, lim))
        pos[k] = p
        yaws[k] = yaw
        pitches[k] = pitch
    return pos, yaws, pitches


def _rect_dist(px, pz, x0, x1, z0, z1):
    dx = np.maximum(np.maximum(x0 - px, 0.0), px - x1)
    dz = np.maximum(np.maximum(z0 - pz, 0.0), pz - z1)
    return np.hypot(dx, dz)


def _place_boxes(rng, n, rmin, rmax, side_lo, side_hi, traj, clearance=0.4):
    """n axis-aligned boxes resting on the floor (y = rmax[1]) whose footprints
    keep `clearance` metres from every camera position."""
    boxes = []
    tries = 0
    while len(boxes) < n:
        tries += 1
        if tries > 200000:
            raise RuntimeError("cannot place boxes")
        s = rng.uniform(side_lo, side_hi, 3)
        x0 = rng.uniform(rmin[0], rmax[0] - s[0])
        z0 = rng.uniform(rmin[2], rmax[2] - s[2])
        if _rect_dist(traj[:, 0], traj[:, 2], x0, x0 + s[0], z0, z0 + s[2]).min() < clearance:
            continue
        boxes.append((np.array([x0, rmax[1] - s[1], z0]), np.array([x0 + s[0], rmax[1], z0 + s[2]])))
    return boxes


def _place_spheres(rng, n, rmin, rmax, r_lo, r_hi, traj, clearance=0.4):
    spheres = []
    tries = 0
    while len(spheres) < n:
        tries += 1
        if tries > 200000:
            raise RuntimeError("cannot place spheres")
        r = rng.uniform(r_lo, r_hi)
        c = rng.uniform(rmin + r, rmax - r)
        if np.linalg.norm(traj - c, axis=1).min() < r + clearance:
            continue
        spheres.append((c, r))
    return spheres


def _room_workload(name, seed, W, H, fx, n_frames, rmin, rmax, n_boxes, box_side,
                   n_spheres, sphere_r, sigma, zero_frac, vs, trunc, cap,
                   table=None, description=""):
    rmin = np.asarray(rmin, np.float64)
    rmax = np.asarray(rmax, np.float64)
    rng = np.random.default_rng([seed, 0])
    margin = 0.4
    traj, yaws, pitches = _random_walk(rng, n_frames, rmin[0] + margin + 0.6,
                                       rmax[0] - margin - 0.6, -0.3, 0.3)
    boxes = _place_boxes(rng, n_boxes, rmin, rmax, box_side[0], box_side[1], traj)
    spheres = _place_spheres(rng, n_spheres, rmin, rmax, sphere_r[0], sphere_r[1], traj) \
        if n_spheres else []
    n_obj = len(boxes) + len(spheres)
    obj_rgb = rng.integers(0, 256, size=(n_obj, 3), dtype=np.uint8)
    face_rgb = rng.integers(0, 256, size=(6, 3), dtype=np.uint8)
    fy = fx
    cx, cy = (W - 1) / 2.0, (H - 1) / 2.0

    def make(i):
        o = traj[i]
        R = _yaw_pitch_rotation(yaws[i], pitches[i])
        t, oid, _ = _cast_scene(o, R, fx, fy, cx, cy, W, H, boxes, spheres, room=(rmin, rmax))
        rgb = np.where((oid >= 0)[..., None], obj_rgb[np.clip(oid, 0, n_obj - 1)],
                       face_rgb[np.clip(-oid - 1, 0, 5)])
        frng = np.random.default_rng([seed, 1, i])
        depth = _finish_depth(t, frng, sigma, zero_frac)
        return _frame(depth, rgb, fx, fy, cx, cy, R, o)

    table = next_pow2(2 * cap) if table is None else table
    wl = Workload(name, W, H, vs, trunc, cap, table, n_frames, make, description)
    wl.trajectory = traj
    wl.boxes = boxes
    wl.spheres = spheres
    return wl


def _room640_workload():
    return _room_workload(
        "room640x480", 3, 640, 480, 525.0, 100, (-3, -1.5, -3), (3, 1.5, 3),
        40, (0.2, 1.2), 0, None, 0.001, 0.10, 0.005, 0.02, 1 << 20,
        description="100 frames 640x480 in a 6x6x3 m room with 40 boxes")


def room_cell(W: int, H: int, fx: float) -> "Workload":
    """The 640 x 480 room's scene and trajectory (same seed, boxes, colours,
    noise and 10% invalid pixels) rendered W x H with focal length fx, for
    the paper's sweep axes: fx proportional to W keeps the field of view and
    the geometry (point count at fixed geometry); fixed fx keeps the angular
    resolution and widens the view (extent at fixed angular resolution).
    At 640 x 480 and fx = 525 its frames are those of room640x480."""
    return _room_workload(
        cell_name(W, H, fx), 3, W, H, float(fx), 100, (-3, -1.5, -3), (3, 1.5, 3),
        40, (0.2, 1.2), 0, None, 0.001, 0.10, 0.005, 0.02, 1 << 20,
        description=f"room640x480's scene rendered {W}x{H}, fx = fy = {fx:g}")


# The sweep cells: (axis, W, H, fx).  "points": fx = 525 W / 640 (same field
# of view, 16x the points from the smallest cell to the largest); "extent":
# fx = 525 (same angle per pixel, the view widens with the image).  The
# smallest cells hold about 17,000 valid points per frame, near the paper's
# smallest cell of 20,000 points.
SWEEP_CELLS = [("points", 160, 120, 131.25), ("points", 320, 240, 262.5), ("points", 640, 480, 525.0),
               ("points", 1280, 960, 1050.0), ("extent", 160, 120, 525.0), ("extent", 320, 240, 525.0),
               ("extent", 1280, 960, 525.0)]


def load_factor_cell(blocks_total: List[int], target: float):
    """The load-factor cells on the room640x480 sequence: pool 2^k (table
    2^(k+1), so the table rule holds) and the longest frame prefix whose
    block count (blocks_total[i]: blocks after frames 0..i, from the stored
    oracle counts) stays within target * table entries.  Returns (pool
    capacity, frames, achieved load factor)."""
    k = 10
    while blocks_total[0] > target * (1 << (k + 1)):
        k += 1
    cap = 1 << k
    n = max(i + 1 for i, t in enumerate(blocks_total) if t <= target * 2 * cap)
    return cap, n, blocks_total[n - 1] / (2 * cap)


LOAD_FACTORS = (0.1, 0.25, 0.5)


def _room1280_workload():
    return _room_workload(
        "room1280x720", 5, 1280, 720, 920.0, 300, (-6, -2, -6), (6, 2, 6),
        150, (0.2, 1.5), 20, (0.2, 0.8), 0.001, 0.0, 0.004, 0.016, 1 << 22,
        table=1 << 24,
        description="300 frames 1280x720 in a 12x12x4 m room, 150 boxes, 20 spheres")


# --------------------------------------------------------------------------
# workload 4 (contention): every point inside a 0.2 m cube
# --------------------------------------------------------------------------
def _cube_workload(seed=4, W=640, H=480, fx=525.0):
    rng = np.random.default_rng([seed, 0])
    cx, cy = (W - 1) / 2.0, (H - 1) / 2.0
    k = 4
    amp = rng.uniform(0.5, 1.0, k)
    amp /= amp.sum()                              # |s| <= 1
    freq = rng.uniform(3.0, 12.0, size=(k, 2)) * rng.choice([-1.0, 1.0], size=(k, 2))
    phase = rng.uniform(0, 2 * math.pi, k)
    colour = _smooth_colour(np.random.default_rng([seed, 2]))

    def s(x, y):
        arg = 2 * math.pi * (x[..., None] * freq[:, 0] + y[..., None] * freq[:, 1]) + phase
        return np.sin(arg) @ amp

    def make(i):
        xn = ((np.arange(W) - cx) / fx)[None, :].repeat(H, 0)
        yn = ((np.arange(H) - cy) / fx)[:, None].repeat(W, 1)
        z = np.full((H, W), 0.14)
        for _ in range(8):                        # Newton on z - 0.14 - 0.01 s(xn z, yn z)
            arg = 2 * math.pi * ((xn * z)[..., None] * freq[:, 0]
                                 + (yn * z)[..., None] * freq[:, 1]) + phase
            val = np.sin(arg) @ amp
            der = (np.cos(arg) * (2 * math.pi) * (xn[..., None] * freq[:, 0]
                                                  + yn[..., None] * freq[:, 1])) @ amp
            z = z - (z - 0.14 - 0.01 * val) / (1.0 - 0.01 * der)
        p = np.stack([xn * z, yn * z, z], -1)
        rgb = _u8(colour(p))
        depth = _finish_depth(z, np.random.default_rng([seed, 1, i]), 0.001, 0.0)
        return _frame(depth, rgb, fx, fx, cx, cy, np.eye(3), np.zeros(3))

    return Workload("cube640x480", W, H, 0.005, 0.02, 65536, 131072, 1, make,
                    "one 640x480 frame, all points inside a 0.2 m cube")


# --------------------------------------------------------------------------
# tiny random frames (brute-force and edge-case tests)
# --------------------------------------------------------------------------
def random_rotation(rng) -> np.ndarray:
    q = rng.normal(size=4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
        [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
        [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)],
    ])


def random_frame(seed, W=7, H=5, depth_range=(0.3, 3.0), invalid_frac=0.0,
                 fx=None, translation_scale=1.0):
    """A frame of independent random depths with a random pose: a tiny,
    structure-free input for exhaustive checks."""
    rng = np.random.default_rng([seed, 7])
    fx = float(rng.uniform(0.6, 1.4) * W) if fx is None else fx
    fy = float(fx * rng.uniform(0.8, 1.25))
    cx = float(rng.uniform(0.3, 0.7) * (W - 1))
    cy = float(rng.uniform(0.3, 0.7) * (H - 1))
    depth = rng.uniform(depth_range[0], depth_range[1], (H, W))
    if invalid_frac > 0:
        depth[rng.random((H, W)) < invalid_frac] = 0.0
    rgb = rng.integers(0, 256, size=(H, W, 3), dtype=np.uint8)
    R = random_rotation(rng)
    t = rng.normal(size=3) * translation_scale
    return _frame(depth.astype(np.float32), rgb, fx, fy, cx, cy, R, t)


# --------------------------------------------------------------------------
# registry
# --------------------------------------------------------------------------
WORKLOADS = {
    "plane64x48": _plane_workload,
    "spherewall320x240": _sphere_wall_workload,
    "spherewall320x240_noisefree": lambda: _sphere_wall_workload(sigma=0.0),
    "room640x480": _room640_workload,
    "cube640x480": _cube_workload,
    "room1280x720": _room1280_workload,
}


def cell_name(W: int, H: int, fx: float) -> str:
    return f"room{W}x{H}_f{fx:g}"


def workload(name: str) -> Workload:
    """A named workload: one of WORKLOADS, or a sweep cell room<W>x<H>_f<fx>."""
    if name in WORKLOADS:
        return WORKLOADS[name]()
    m = re.fullmatch(r"room(\d+)x(\d+)_f([0-9.]+)", name)
    if m:
        return room_cell(int(m.group(1)), int(m.group(2)), float(m.group(3)))
    raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)} and room<W>x<H>_f<fx>")


# How the benchmark splits each workload into calls (tsdf_integrate_batch
# of a call's frames): contiguous (first, end) frame ranges.  The stored
# oracle counts hold the compulsory traffic of exactly these calls.
BENCH_CALLS = {
    "plane64x48": [(0, 1)],
    "spherewall320x240": [(0, 10)],
    "cube640x480": [(0, 1)],
    "room640x480": [(0, 100)],
    "room1280x720": [(0, 100), (100, 200), (200, 300)],
}
