"""The seeded input generator: determinism and the scene facts the pins use."""
import math

import numpy as np
import pytest

from hash_table_amd import scenes


def test_plane_frame_is_exact():
    f = scenes.workload("plane64x48").frame(0)
    assert f.depth.dtype == np.float32 and f.depth.shape == (48, 64)
    assert np.all(f.depth == 1.0)
    assert f.rgb.dtype == np.uint8 and f.rgb.shape == (48, 64, 3)
    assert np.array_equal(f.R, np.eye(3, dtype=np.float32)) and not f.t.any()
    assert (f.fx, f.fy, f.cx, f.cy) == (50.0, 50.0, 32.0, 24.0)


@pytest.mark.parametrize("name,idx", [("spherewall320x240", 3), ("room640x480", 7), ("cube640x480", 0)])
def test_seeded_determinism(name, idx):
    a = scenes.workload(name).frame(idx)
    b = scenes.workload(name).frame(idx)
    assert scenes.frame_digest([a]) == scenes.frame_digest([b])


def test_sphere_depth_is_analytic():
    wl = scenes.workload("spherewall320x240_noisefree")
    f = wl.frame(0)                           # camera at the origin looking along +z
    H, W = f.depth.shape
    u, v = np.meshgrid(np.arange(W), np.arange(H))
    xn = (u - f.cx) / f.fx
    yn = (v - f.cy) / f.fy
    # sphere |p - (0,0,1.5)| = 0.5 with p = z (xn, yn, 1)
    a = xn ** 2 + yn ** 2 + 1
    b = -3.0
    c = 1.5 ** 2 - 0.25
    disc = b * b - 4 * a * c
    z = np.where(disc >= 0, (-b - np.sqrt(np.maximum(disc, 0))) / (2 * a), 3.0)
    assert np.abs(f.depth - z).max() < 1e-6
    assert abs(f.depth[H // 2, W // 2] - 1.0) < 1e-3


def test_room_statistics():
    wl = scenes.workload("room640x480")
    f = wl.frame(0)
    valid = f.depth > 0
    assert 0.85 < valid.mean() < 0.95                     # 10 % of pixels zeroed
    assert f.depth[valid].min() > 0.3 and f.depth.max() < 9.0
    R = f.R.astype(np.float64)
    assert np.abs(R @ R.T - np.eye(3)).max() < 1e-6
    # camera stays inside the room and keeps clear of the boxes
    traj = wl.trajectory
    assert np.all(np.abs(traj[:, 0]) < 2.6) and np.all(np.abs(traj[:, 2]) < 2.6)
    for bmin, bmax in wl.boxes:
        dx = np.maximum(np.maximum(bmin[0] - traj[:, 0], 0), traj[:, 0] - bmax[0])
        dz = np.maximum(np.maximum(bmin[2] - traj[:, 2], 0), traj[:, 2] - bmax[2])
        assert np.hypot(dx, dz).min() >= 0.4
    # a smooth walk: at most a few cm and ~1 degree between frames
    steps = np.linalg.norm(np.diff(traj, axis=0), axis=1)
    assert steps.max() < 0.05


def test_cube_points_inside_cube():
    f = scenes.workload("cube640x480").frame(0)
    d = f.depth
    assert d.min() > 0.12 and d.max() < 0.16
    H, W = d.shape
    u, v = np.meshgrid(np.arange(W), np.arange(H))
    x = (u - f.cx) / f.fx * d
    y = (v - f.cy) / f.fy * d
    assert x.max() - x.min() < 0.2 and y.max() - y.min() < 0.2 and d.max() - d.min() < 0.2


def test_random_frame_pose_is_rotation():
    f = scenes.random_frame(3)
    R = f.R.astype(np.float64)
    assert abs(np.linalg.det(R) - 1) < 1e-6
    assert np.abs(R @ R.T - np.eye(3)).max() < 1e-6


def test_next_pow2():
    assert [scenes.next_pow2(n) for n in (1, 2, 3, 8192, 8193)] == [1, 2, 4, 8192, 16384]
    assert scenes.next_pow2(2 * 4096) == 8192
