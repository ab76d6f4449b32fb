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
