"""The rounding margin behind allocate's band test on a stepped sdf (no GPU).

Allocate decides the band on d - zc stepped from an exact evaluation at a
chunk's first cell (one subtraction per step of the pose's depth-axis entry
times vs) wherever that value lies further than a margin m from +-trunc, and
takes the exact test inside it.  Its decisions are the exact test's if and
only if |exact - stepped| <= m at every cell of a chunk (at most 31 steps).
This models both in float32 (numpy rounds every operation to float32 and
fuses none, as the kernel is compiled) over random poses, cameras from the
origin out to 300 m, random depths and random step sequences, and checks the
bound at every cell.  The margin is the kernel's:
m = 2^-20 (r (sum|X| + sum|t| + 80 vs) + d + 2 |sdf0|) + 2^-22 trunc.
"""
from __future__ import annotations

import numpy as np
import pytest

f32 = np.float32


def _rotations(rng, n):
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    R = np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w),
                  2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w),
                  2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)], axis=1)
    return R.astype(np.float32)                      # (n, 9), row-major


def _exact_sdf(cx, cy, cz, d, r2, r5, r8, t0, t1, t2, vs):
    """The centre test's sdf in float32, in the kernel's operation order."""
    c0, c1, c2 = cx * vs, cy * vs, cz * vs
    zc = (r2 * (c0 - t0) + r5 * (c1 - t1)) + r8 * (c2 - t2)
    return d - zc


@pytest.mark.parametrize("dist", [0.0, 3.0, 40.0, 300.0])
@pytest.mark.parametrize("vs,trunc", [(0.005, 0.02), (0.01, 0.04), (2.0 ** -7, 2.0 ** -5)])
def test_stepped_sdf_stays_within_margin(dist, vs, trunc):
    rng = np.random.default_rng([int(dist), int(vs * 1e6), 5])
    n = 20000
    R = _rotations(rng, n)
    r2, r5, r8 = R[:, 2], R[:, 5], R[:, 8]
    t = (rng.normal(size=(n, 3)) + dist).astype(np.float32)
    t0, t1, t2 = t[:, 0], t[:, 1], t[:, 2]
    d = rng.uniform(0.2, 8.0, size=n).astype(np.float32)
    vs, trunc = f32(vs), f32(trunc)
    # a chunk's first cell: a voxel near the camera's band, centre k + 1/2 (exact)
    k = np.floor(t / vs + rng.uniform(-2.0, 2.0, size=(n, 3)) / vs).astype(np.int64)
    x = [(k[:, a] + 0.5).astype(np.float32) for a in range(3)]
    sdf0 = _exact_sdf(x[0], x[1], x[2], d, r2, r5, r8, t0, t1, t2, vs)
    # the kernel's margin
    r_max = np.maximum(np.maximum(np.abs(r2), np.abs(r5)), np.maximum(np.abs(r8), f32(1.0)))
    t_abs = (np.abs(t0) + np.abs(t1)) + np.abs(t2)
    xs = (np.abs(x[0] * vs) + np.abs(x[1] * vs)) + np.abs(x[2] * vs)
    m = f32(2.0 ** -20) * ((r_max * ((xs + t_abs) + f32(80.0) * vs) + np.abs(d)) + f32(2.0) * np.abs(sdf0)) + \
        f32(2.0 ** -22) * trunc
    # steps: each ray walks 31 unit steps along random axes, one direction per axis
    sgn = rng.choice(np.array([-1.0, 1.0], np.float32), size=(n, 3))
    dl = [(sgn[:, 0] * r2) * vs, (sgn[:, 1] * r5) * vs, (sgn[:, 2] * r8) * vs]
    sa = sdf0.copy()
    worst = 0.0
    nonzero = 0
    for _ in range(31):
        axis = rng.integers(0, 3, size=n)
        for a in range(3):
            sel = axis == a
            x[a] = np.where(sel, x[a] + sgn[:, a], x[a])
            sa = np.where(sel, sa - dl[a], sa)
        exact = _exact_sdf(x[0], x[1], x[2], d, r2, r5, r8, t0, t1, t2, vs)
        err = np.abs(exact.astype(np.float64) - sa.astype(np.float64))
        assert np.all(err <= m.astype(np.float64)), (float(err.max()), float(m[np.argmax(err - m)]))
        worst = max(worst, float(np.max(err / m)))
        nonzero += int(np.count_nonzero(err))
    assert x[0].dtype == np.float32 and sa.dtype == np.float32
    # the model exercises rounding (the stepped value does drift from the exact one)
    assert nonzero > 0
    assert worst < 1.0
