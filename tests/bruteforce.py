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


def hidden_by_depth(frame, K, vs, tr, eps_px=1e-4, eps_z=1e-5):
    """The reprojection reading of the occlusion test, in float64, for cells K
    (n x 3): each centre, in camera coordinates, projected to its nearest
    pixel; hidden iff that pixel is in the image with a valid depth D and the
    centre lies more than trunc behind it.  Returns (hidden, tie) per cell;
    tie marks a projection within eps_px of a pixel edge or a depth gap
    within eps_z of trunc, which float32 may decide either way."""
    R = frame.R.astype(np.float64)
    t = frame.t.astype(np.float64)
    H, W = frame.depth.shape
    cam = ((K + 0.5) * vs - t) @ R              # rows: (xc, yc, zc)
    zc = cam[:, 2]
    front = zc > 0
    zs = np.where(front, zc, 1.0)
    uf = cam[:, 0] / zs * float(frame.fx) + float(frame.cx) + 0.5
    vf = cam[:, 1] / zs * float(frame.fy) + float(frame.cy) + 0.5
    inside = front & (uf >= 0) & (uf < W) & (vf >= 0) & (vf < H)
    iu = np.clip(np.floor(uf), 0, W - 1).astype(np.int64)
    iv = np.clip(np.floor(vf), 0, H - 1).astype(np.int64)
    D = frame.depth[iv, iu].astype(np.float64)
    valid = inside & np.isfinite(D) & (D > 0)
    gap = zc - D
    hidden = valid & (gap > tr)
    edge = lambda x: np.abs(x - np.round(x)) < eps_px
    tie = front & (edge(uf) | edge(vf) | (valid & (np.abs(gap - tr) < eps_z)))
    return hidden, tie


def crossed_cells(frame, u, v, voxel_size, trunc, eps=1e-3):
    """Number of unit cells the closed band segment of pixel (u, v) crosses
    (length of segment inside the cell > eps voxels), and whether any cell is
    too close to call (the segment grazing a cell edge or face).  None for an
    invalid or near pixel."""
    r = _segment_cells(frame, u, v, voxel_size, trunc, eps)
    if r is None:
        return None, False
    K, crosses, tie, _, _, _ = r
    return int(crosses.sum()), tie


def _segment_cells(frame, u, v, voxel_size, trunc, eps):
    """The cells of the band segment's bounding box (plus one of margin),
    which of them the segment crosses, and whether any is a tie; with the
    point's depth, the pose and the float32 voxel size / trunc."""
    vs = float(np.float32(voxel_size))
    tr = float(np.float32(trunc))
    d = float(frame.depth[v, u])
    if not np.isfinite(d) or d <= tr:
        return None
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
    return K, crosses, tie, overlap_vox, d, (vs, tr, R, t)


def point_voxels(frame, u, v, voxel_size, trunc, eps=1e-3, eps_sdf=1e-5, reproject=False):
    """Return (voxels, tie): voxels maps (kx, ky, kz) -> (tsdf, r, g, b) for the
    kept voxels of pixel (u, v); tie is True if any decision was too close to
    call in float32.  Returns (None, False) for an invalid/near pixel.  With
    reproject, kept cells must also pass hidden_by_depth against the frame's
    depth image, and the result is (voxels, tie_cells): the set of cells
    whose decision is a tie (the others are exact)."""
    r = _segment_cells(frame, u, v, voxel_size, trunc, eps)
    if r is None:
        return None, False
    K, crosses, tie, overlap_vox, d, (vs, tr, R, t) = r
    c = (K + 0.5) * vs
    zc = (c - t) @ R[:, 2]
    sdf = d - zc
    kept = crosses & (sdf >= -tr) & (sdf <= tr)
    cell_tie = crosses & ((np.abs(sdf - tr) < eps_sdf) | (np.abs(sdf + tr) < eps_sdf))
    if reproject:
        # per cell: a walk tie (the segment grazing a cell) makes every cell
        # of the point uncertain; a band or projection tie only that cell
        hid, ptie = hidden_by_depth(frame, K, vs, tr)
        cell_tie |= kept & ptie
        kept &= ~hid
        if tie:                                    # every cell the segment may touch
            cell_tie |= overlap_vox > -eps
    tie |= bool(np.any(cell_tie))
    rgb = frame.rgb[v, u].astype(np.float64) / 255.0
    out = {}
    for k, s in zip(map(tuple, K[kept]), sdf[kept]):
        out[k] = (s / tr, rgb[0], rgb[1], rgb[2])
    if reproject:
        return out, {tuple(k) for k in K[cell_tie]}
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
