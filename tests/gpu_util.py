"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare
with the oracle."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

import oracle
from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import pipeline as PL

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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
    proj.radii.copy_(torch.from_numpy(np.ascontiguousarray(P.radii, np.int32)))
    proj.depth.copy_(torch.from_numpy(P.dkey))
    proj.rec.copy_(torch.from_numpy(rec))
    return proj


def gpu_forward(scene, cam, rp=None, capacity=0):
    """Project, bin and render one view on the GPU.  Returns the TrainStep holding the buffers."""
    params = PL.GaussianParams.from_scene(scene, DEV)
    step = PL.TrainStep(params, cam.width, cam.height, DEV, raster=rp, capacity=capacity, plain=True)
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


# Where one comparison's statistics are appended (one JSON object per line), so that a GPU
# run reports the tie and mismatch counts of every image it compared (GS_TIE_LOG overrides).
TIE_LOG = os.environ.get("GS_TIE_LOG", os.path.join(ROOT, "tests", "logs", "image_compare_stats.jsonl"))


def _record(stats):
    try:
        os.makedirs(os.path.dirname(TIE_LOG), exist_ok=True)
        with open(TIE_LOG, "a") as fh:
            fh.write(json.dumps(stats) + "\n")
    except OSError:
        pass


def compare_images(gpu_c, gpu_t, orc_c, orc_t, tie, gpu_n=None, orc_n=None, tol=1e-4, max_excused_frac=1e-5,
                   label=None):
    """Image parity.  A pixel fails if its colour or final transmittance differs from the
    oracle's by more than tol, or (with gpu_n / orc_n) its traversal count N_p differs.  The
    oracle flags as ties the pixels where a decision (alpha against alpha_min, T against
    theta_T, a marginal cull) lies within its rounding margin; a failing pixel is excused
    only if it is flagged, and the excused pixels may be at most max_excused_frac of the
    image.  Every other pixel must pass, N_p included.  The counts are logged and recorded."""
    gpu_c = np.asarray(gpu_c).reshape(-1, 3)
    orc_c = np.asarray(orc_c).reshape(-1, 3)
    gpu_t, orc_t = np.asarray(gpu_t).reshape(-1), np.asarray(orc_t).reshape(-1)
    tie = np.asarray(tie, bool).reshape(-1)
    dc = np.abs(gpu_c.astype(np.float64) - orc_c).max(axis=-1)
    dt = np.abs(gpu_t.astype(np.float64) - orc_t)
    bad = (dc > tol) | (dt > tol)
    n_mism = 0
    if gpu_n is not None:
        nm = np.asarray(gpu_n).reshape(-1) != np.asarray(orc_n).reshape(-1)
        n_mism = int(nm.sum())
        bad |= nm
    excused = bad & tie
    unexcused = bad & ~tie
    keep = ~excused
    n = int(tie.size)
    stats = dict(label=label or os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], n=n,
                 flagged=int(tie.sum()), excused=int(excused.sum()), unexcused=int(unexcused.sum()),
                 ntrav_mismatch=n_mism,
                 max_color=float(dc[keep].max()) if keep.any() else 0.0,
                 max_t=float(dt[keep].max()) if keep.any() else 0.0,
                 excused_max=float(max(dc[excused].max(), dt[excused].max())) if excused.any() else 0.0)
    _record(stats)
    log(f"  image compare {stats}")
    assert stats["unexcused"] == 0, stats
    assert stats["excused"] <= int(max_excused_frac * n), stats
    return stats


def compare_projection(proj, P, ulps=2):
    """GPU projected records against the oracle's float32 record: cull decisions and
    depth keys bit-identical (outside marginal culls), radii equal, means within `ulps`
    float32 ulps, conic within 1e-6 of its largest entry, colour within 2e-6, opacity within
    1 ulp (its log2 in the raster record within what that ulp and one rounding allow).  Checked in the raster record, which
    also carries the index and the radii (a culled Gaussian's record is zero apart from its
    index), and in the plain record planes where the projection holds them."""
    radii = proj.radii.cpu().numpy()
    vis_g = (radii[:, 0] > 0) & (radii[:, 1] > 0)
    marg = P.marginal.astype(bool)
    assert np.array_equal(vis_g[~marg], P.vis[~marg].astype(bool))
    dk = proj.depth.cpu().numpy()
    assert np.array_equal(dk.view(np.uint32), P.dkey.view(np.uint32)), "depth keys must be bit-identical"
    v = vis_g & P.vis.astype(bool)
    assert np.array_equal(radii[v], P.radii[v])
    n = radii.shape[0]
    grec = proj.rec.cpu().numpy()
    bits = grec.view(np.uint32)
    assert np.array_equal(bits[:, 9], np.arange(n, dtype=np.uint32)), "record index"
    assert np.array_equal(bits[:, 10:12].view(np.int32), radii), "record radii"
    culled = ~vis_g
    assert not bits[culled][:, [0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 11]].any(), "a culled record must be zero"
    rec = P.rec[v]
    g = grec[v]
    stats = dict(visible=int(v.sum()), marginal=int(marg.sum()),
                 mean_ulps=int(ulp_diff(g[:, :2], rec[:, :2].astype(np.float32)).max()) if v.any() else 0)
    assert stats["mean_ulps"] <= ulps, stats
    if v.any():
        # conic: both sides invert Sigma2D in double; allow a few ulps of the larger entry
        l2e = 1.4426950408889634
        want = rec[:, 2:5] * np.array([-0.5 * l2e, -l2e, -0.5 * l2e])
        scale = np.abs(want).max(axis=1, keepdims=True)
        assert (np.abs(g[:, 2:5] - want) / scale).max() < 1e-6
        # log2 of the float32 opacity, rounded to float32: one ulp of o moves it by at most
        # 1.8e-7, its own rounding by half an ulp of the result
        lo = np.log2(rec[:, 5].astype(np.float32).astype(np.float64))
        tol = 1.8e-7 + 2 * np.spacing(np.abs(lo).astype(np.float32)).astype(np.float64)
        assert (np.abs(g[:, 5] - lo) <= tol).all()
        assert np.abs(g[:, 6:9] - rec[:, 6:9]).max() < 2e-6 * max(1.0, np.abs(rec[:, 6:9]).max())
    if proj.means2d is not None:
        m2 = proj.means2d.cpu().numpy().T[v]
        co = proj.conic_opacity.cpu().numpy().T[v]
        col = proj.color.cpu().numpy().T[v]
        assert np.array_equal(m2, g[:, :2]), "plain means equal the record's"
        assert np.array_equal(col, g[:, 6:9]), "plain colour equals the record's"
        assert ulp_diff(co[:, 3], rec[:, 5].astype(np.float32)).max() <= 1
        scale = np.abs(rec[:, 2:5]).max(axis=1, keepdims=True)
        assert (np.abs(co[:, :3] - rec[:, 2:5]) / scale).max() < 1e-6
    return stats
