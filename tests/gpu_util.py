"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare
with the oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import pipeline as PL

DEV = "cuda"


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def oracle_params(rp: B.RasterParams) -> oracle.Params:
    return oracle.Params(alpha_min=float(np.float32(rp.alpha_min)), alpha_max=float(np.float32(rp.alpha_max)),
                         t_min=float(np.float32(rp.t_min)), near_z=float(np.float32(0.01)),
                         depth_lo=float(np.float32(rp.depth_lo)), depth_hi=float(np.float32(rp.depth_hi)))


def synthetic_projection(m2, r, d):
    """Projected records for the binning stage alone: means, radii, depth keys, and the
    raster records' u, v and box half-extents (conic zero: every quadrant test passes)."""
    n = d.numel()
    proj = PL.Projection(max(n, 1), DEV)
    if n:
        proj.means2d[:n].copy_(m2.to(DEV))
        proj.radii[:n].copy_(r.to(DEV))
        proj.depth[:n].copy_(d.to(DEV))
        proj.rec[:n, 0:2].copy_(m2.to(DEV))
        proj.rec[:n, 10:12].copy_(r.to(DEV).view(torch.float32))
    return proj


def oracle_projection(P, n):
    """The oracle's float32 projected records in the GPU layout (the raster record formed
    as the projection forms it: conic scaled for exp2, log2 of the float32 opacity)."""
    l2e = 1.4426950408889634
    rec = np.zeros((n, 12), np.float32)
    rec[:, 0:2] = P.rec[:, 0:2]
    rec[:, 2] = -0.5 * l2e * P.rec[:, 2]
    rec[:, 3] = -l2e * P.rec[:, 3]
    rec[:, 4] = -0.5 * l2e * P.rec[:, 4]
    with np.errstate(divide="ignore"):
        rec[:, 5] = np.log2(P.rec[:, 5].astype(np.float32).astype(np.float64))
    rec[:, 6:9] = P.rec[:, 6:9]
    rec[:, 9] = np.arange(n, dtype=np.uint32).view(np.float32)
    rec[:, 10:12] = np.ascontiguousarray(P.radii, np.int32).view(np.float32)
    proj = PL.Projection(n, DEV)
    proj.means2d.copy_(torch.from_numpy(P.rec[:, :2].astype(np.float32)))
    proj.radii.copy_(torch.from_numpy(np.ascontiguousarray(P.radii, np.int32)))
    proj.depth.copy_(torch.from_numpy(P.dkey))
    co = np.zeros((n, 4), np.float32)
    co[:, :3] = P.rec[:, 2:5]
    co[:, 3] = P.rec[:, 5]
    proj.conic_opacity.copy_(torch.from_numpy(co))
    proj.color.copy_(torch.from_numpy(P.rec[:, 6:9].astype(np.float32)))
    proj.rec.copy_(torch.from_numpy(rec))
    return proj


def gpu_forward(scene, cam, rp=None, capacity=0):
    """Project, bin and render one view on the GPU.  Returns the TrainStep holding the buffers."""
    params = PL.GaussianParams.from_scene(scene, DEV)
    step = PL.TrainStep(params, cam.width, cam.height, DEV, raster=rp, capacity=capacity)
    step.forward(B.camera_from(cam))
    torch.cuda.synchronize()
    return step


def ulp_diff(a, b):
    """Distance in float32 units in the last place (same sign assumed close to each other)."""
    a = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / den if den > 0 else np.linalg.norm(a - b)


def compare_images(gpu_c, gpu_t, orc_c, orc_t, tie, tol=1e-4, tie_tol=1e-2, max_tie_frac=5e-3):
    """Max |difference| outside tie pixels must be <= tol; tie pixels (a decision within
    rounding distance of its threshold) are bounded by tie_tol and counted."""
    dc = np.abs(gpu_c.astype(np.float64) - orc_c).max(axis=-1)
    dt = np.abs(gpu_t.astype(np.float64) - orc_t)
    ok = ~tie
    stats = dict(max_color=float(dc[ok].max()) if ok.any() else 0.0, max_t=float(dt[ok].max()) if ok.any() else 0.0,
                 ties=int(tie.sum()), n=int(tie.size),
                 tie_max=float(max(dc[tie].max(), dt[tie].max())) if tie.any() else 0.0)
    assert stats["max_color"] <= tol and stats["max_t"] <= tol, stats
    assert stats["ties"] <= max(2, max_tie_frac * tie.size), stats
    assert stats["tie_max"] <= tie_tol, stats
    return stats
