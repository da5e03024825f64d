"""Brute-force band enumeration in float64, independent of any voxel walk.

For one depth point it lists every voxel whose closed band segment crosses the
half-open cell and whose centre passes the occlusion/band test, by testing
every cell of the segment's bounding box (plus one cell of margin) in double
precision.  Cells that sit within `eps` of a decision (the segment grazing a
cell edge, or a centre within `eps_sdf` of +-trunc) are reported as ties: the
float32 walk may decide them either way, so callers skip such points.

The quantities follow the method of "What Irregularity Costs" (section 3: the
band walk over the voxels a point touches, weighted sums; section 4: signed
distance at the voxel centre); the camera model, band segment and occlusion
test are the readings both implementations use.
"""
from __future__ import annotations

import numpy as np


def point_voxels(frame, u, v, voxel_size, trunc, eps=1e-3, eps_sdf=1e-5):
    """Return (voxels, tie): voxels maps (kx, ky, kz) -> (tsdf, r, g, b) for the
    kept voxels of pixel (u, v); tie is True if any decision was too close to
    call in float32.  Returns (None, False) for an invalid/near pixel."""
    vs = float(np.float32(voxel_size))
    tr = float(np.float32(trunc))
    d = float(frame.depth[v, u])
    if not np.isfinite(d) or d <= tr:
        return None, False
    R = frame.R.astype(np.float64)
    t = frame.t.astype(np.float64)
    xn = (u - float(frame.cx)) / float(frame.fx)
    yn = (v - float(frame.cy)) / float(frame.fy)
    ray = np.array([xn, yn, 1.0])
    gA = (R @ (ray * (d - tr)) + t) / vs
    gB = (R @ (ray * (d + tr)) + t) / vs
    direction = gB - gA
    seg_len = float(np.linalg.norm(direction))
    lo = np.floor(np.minimum(gA, gB)).astype(np.int64) - 1
    hi = np.floor(np.maximum(gA, gB)).astype(np.int64) + 1
    axes = [np.arange(lo[i], hi[i] + 1) for i in range(3)]
    K = np.stack(np.meshgrid(*axes, indexing="ij"), -1).reshape(-1, 3)

    # parameter interval [s_lo, s_hi] of the segment inside each cell, per axis
    s_lo = np.zeros(K.shape)
    s_hi = np.ones(K.shape)
    grazing = np.zeros(K.shape[0], bool)
    for i in range(3):
        if abs(direction[i]) > 1e-12:
            a = (K[:, i] - gA[i]) / direction[i]
            b = (K[:, i] + 1 - gA[i]) / direction[i]
            s_lo[:, i] = np.minimum(a, b)
            s_hi[:, i] = np.maximum(a, b)
        else:
            inside = (K[:, i] <= gA[i]) & (gA[i] < K[:, i] + 1)
            s_lo[:, i] = np.where(inside, 0.0, 2.0)
            s_hi[:, i] = np.where(inside, 1.0, -1.0)
            near = (np.abs(gA[i] - K[:, i]) < eps) | (np.abs(gA[i] - K[:, i] - 1) < eps)
            grazing |= near
    overlap = np.minimum(1.0, s_hi.min(1)) - np.maximum(0.0, s_lo.max(1))
    overlap_vox = overlap * seg_len          # length of segment inside the cell, voxels
    crosses = overlap_vox > eps
    tie = bool(np.any((np.abs(overlap_vox) <= eps) | (grazing & (overlap_vox > -eps))))

    c = (K + 0.5) * vs
    zc = (c - t) @ R[:, 2]
    sdf = d - zc
    kept = crosses & (sdf >= -tr) & (sdf <= tr)
    tie |= bool(np.any(crosses & ((np.abs(sdf - tr) < eps_sdf) | (np.abs(sdf + tr) < eps_sdf))))
    rgb = frame.rgb[v, u].astype(np.float64) / 255.0
    out = {}
    for k, s in zip(map(tuple, K[kept]), sdf[kept]):
        out[k] = (s / tr, rgb[0], rgb[1], rgb[2])
    return out, tie


def frame_voxels(frame, voxel_size, trunc, **kw):
    """Aggregate brute-force contributions of every pixel of a frame.
    Returns (sums, ties): sums maps voxel -> [tsdf, weight, r, g, b]."""
    sums = {}
    ties = 0
    H, W = frame.depth.shape
    for v in range(H):
        for u in range(W):
            vox, tie = point_voxels(frame, u, v, voxel_size, trunc, **kw)
            if vox is None:
                continue
            ties += int(tie)
            for k, (ts, r, g, b) in vox.items():
                acc = sums.setdefault(k, [0.0, 0.0, 0.0, 0.0, 0.0])
                acc[0] += ts
                acc[1] += 1.0
                acc[2] += r
                acc[3] += g
                acc[4] += b
    return sums, ties
