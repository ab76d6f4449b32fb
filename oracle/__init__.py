"""CPU oracle for the Gaussian-splatting training step (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does.  ``gs_oracle.c`` holds the arithmetic; this module
only marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.c")
_LIB = os.path.join(_HERE, "libgs_oracle.so")
_lib = None

G_FIELDS = ("u", "v", "A", "B", "C", "opacity", "r", "g", "b")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (double precision, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fno-fast-math",
                               "-ffp-contract=off", "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


@dataclass
class Params:
    alpha_min: float = float(np.float32(1.0 / 255.0))
    alpha_max: float = float(np.float32(0.99))
    t_min: float = float(np.float32(1e-4))
    near_z: float = float(np.float32(0.01))
    depth_lo: float = 0.0
    depth_hi: float = float("inf")


def _p(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _np(x, dtype=np.float32):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def _cam(cam):
    vm = _np(cam.viewmat).reshape(16)
    intr = np.array([cam.fx, cam.fy, cam.cx, cam.cy], dtype=np.float32)
    return vm, intr


@dataclass
class Projected:
    vis: np.ndarray       # int32 [n]
    rec: np.ndarray       # float64 [n][9]  (u, v, A, B, C, o, r, g, b)
    dkey: np.ndarray      # float32 [n]
    radii: np.ndarray     # int32 [n][2]
    marginal: np.ndarray  # uint8 [n]
    width: int
    height: int


def _scene_arrays(scene):
    return [_p(_np(a, np.float64), np.float64) for a in
            (scene.means, scene.log_scales, scene.quats, scene.opacity_logits, scene.sh)]


def _cam64(cam):
    vm, intr = _cam(cam)
    return _p(vm.astype(np.float64), np.float64), _p(intr.astype(np.float64), np.float64)


def project(scene, cam, params: Params = Params(), round_record: bool = True) -> Projected:
    """Project every Gaussian.  round_record rounds the 2D record to float32 (the
    method's record); without it the record is exact (finite-difference checks)."""
    L = lib()
    n = scene.n
    arrs = _scene_arrays(scene)
    (vm, pvm), (intr, pin) = _cam64(cam)
    vis = np.zeros(n, np.int32)
    rec = np.zeros((n, 9), np.float64)
    dkey = np.zeros(n, np.float32)
    radii = np.zeros((n, 2), np.int32)
    marg = np.zeros(n, np.uint8)
    f = L.orc_project
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 7 + [
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_float, ctypes.c_float,
        ctypes.c_int] + [ctypes.c_void_p] * 5
    rc = f(n, scene.sh_degree, *[a[1] for a in arrs], pvm, pin, cam.width, cam.height,
           params.near_z, params.alpha_min, params.depth_lo, params.depth_hi, int(round_record),
           vis.ctypes.data, rec.ctypes.data, dkey.ctypes.data, radii.ctypes.data, marg.ctypes.data)
    assert rc == 0
    return Projected(vis, rec, dkey, radii, marg, cam.width, cam.height)


def all_pixels(width, height):
    ys, xs = np.meshgrid(np.arange(height, dtype=np.int32), np.arange(width, dtype=np.int32), indexing="ij")
    return np.stack([xs.reshape(-1), ys.reshape(-1)], axis=1).copy()


def render(P: Projected, params: Params = Params(), pixels=None, literal=False):
    """Returns (color [npix,3] f64, t_final [npix] f64, n_trav [npix] i32, tie [npix] bool).
    With pixels=None the whole image is rendered and outputs are shaped [H,W,...]."""
    L = lib()
    full = pixels is None
    pix = all_pixels(P.width, P.height) if full else np.ascontiguousarray(pixels, np.int32)
    npix = pix.shape[0]
    col = np.zeros((npix, 3), np.float64)
    tf = np.zeros(npix, np.float64)
    nt = np.zeros(npix, np.int32)
    tie = np.zeros(npix, np.uint8)
    f = L.orc_render
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64] + [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_int] + [
        ctypes.c_float] * 3 + [ctypes.c_int, ctypes.c_int64] + [ctypes.c_void_p] * 5
    n = P.vis.shape[0]
    rc = f(n, P.vis.ctypes.data, P.rec.ctypes.data, P.dkey.ctypes.data, P.radii.ctypes.data,
           P.marginal.ctypes.data, P.width, P.height, params.alpha_min, params.alpha_max, params.t_min,
           int(bool(literal)), npix, pix.ctypes.data, col.ctypes.data, tf.ctypes.data, nt.ctypes.data,
           tie.ctypes.data)
    assert rc == 0
    tie = tie.astype(bool)
    if full:
        H, W = P.height, P.width
        return col.reshape(H, W, 3), tf.reshape(H, W), nt.reshape(H, W), tie.reshape(H, W)
    return col, tf, nt, tie


def raster_backward(P: Projected, G, GT=None, params: Params = Params(), pixels=None):
    """Screen-space gradients [9][n] (float64), summed over the given pixels
    (all pixels by default).  G: [npix,3] or [H,W,3]; GT: [npix] / [H,W] or None."""
    L = lib()
    pix = all_pixels(P.width, P.height) if pixels is None else np.ascontiguousarray(pixels, np.int32)
    npix = pix.shape[0]
    G = np.ascontiguousarray(np.asarray(G, np.float64).reshape(npix, 3))
    gt_ptr = None
    if GT is not None:
        GT = np.ascontiguousarray(np.asarray(GT, np.float64).reshape(npix))
        gt_ptr = GT.ctypes.data
    n = P.vis.shape[0]
    out = np.zeros((9, n), np.float64)
    f = L.orc_raster_backward
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64] + [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_int] + [
        ctypes.c_float] * 3 + [ctypes.c_int64] + [ctypes.c_void_p] * 4
    rc = f(n, P.vis.ctypes.data, P.rec.ctypes.data, P.dkey.ctypes.data, P.radii.ctypes.data,
           P.width, P.height, params.alpha_min, params.alpha_max, params.t_min, npix, pix.ctypes.data,
           G.ctypes.data, gt_ptr, out.ctypes.data)
    assert rc == 0
    return out


def project_backward(scene, cam, grads2d, params: Params = Params(), round_record: bool = True):
    """Gradients of the 3D parameters (float64, same plane layout as the scene)."""
    L = lib()
    n, K = scene.n, scene.k_sh
    arrs = _scene_arrays(scene)
    (vm, pvm), (intr, pin) = _cam64(cam)
    g2 = np.ascontiguousarray(grads2d, np.float64)
    out = dict(means=np.zeros((3, n)), log_scales=np.zeros((3, n)), quats=np.zeros((4, n)),
               opacity_logits=np.zeros(n), sh=np.zeros((3 * K, n)))
    f = L.orc_project_backward
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 7 + [
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_float, ctypes.c_float,
        ctypes.c_int] + [ctypes.c_void_p] * 6
    rc = f(n, scene.sh_degree, *[a[1] for a in arrs], pvm, pin, cam.width, cam.height, params.near_z,
           params.alpha_min, params.depth_lo, params.depth_hi, int(round_record), g2.ctypes.data,
           out["means"].ctypes.data, out["log_scales"].ctypes.data, out["quats"].ctypes.data,
           out["opacity_logits"].ctypes.data, out["sh"].ctypes.data)
    assert rc == 0
    return out


def bin_f32(means2d, radii, depth, width, height, cap=None):
    """Bit-exact binning from float projected inputs.
    Returns (tiles_touched [n] i32, keys [K] u64, ids [K] u32, ranges [T+1] i32)."""
    L = lib()
    m2 = _np(means2d, np.float32).reshape(-1, 2)
    r = _np(radii, np.int32).reshape(-1, 2)
    d = _np(depth, np.float32).reshape(-1)
    n = d.shape[0]
    tx, ty = (width + 15) // 16, (height + 15) // 16
    tt = np.zeros(n, np.int32)
    f = L.orc_bin_f32
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    ranges = np.zeros(tx * ty + 1, np.int32)
    K = f(n, m2.ctypes.data, r.ctypes.data, d.ctypes.data, width, height, tt.ctypes.data, 0, None, None,
          ranges.ctypes.data)
    keys = np.zeros(max(K, 1), np.uint64)
    ids = np.zeros(max(K, 1), np.uint32)
    K2 = f(n, m2.ctypes.data, r.ctypes.data, d.ctypes.data, width, height, tt.ctypes.data, K,
           keys.ctypes.data, ids.ctypes.data, ranges.ctypes.data)
    assert K2 == K
    return tt, keys[:K], ids[:K], ranges


def loss_l1(color, target):
    L = lib()
    c = _np(color, np.float32).reshape(-1)
    t = _np(target, np.float32).reshape(-1)
    assert c.shape == t.shape and c.size % 3 == 0
    G = np.zeros(c.size, np.float64)
    f = L.orc_loss_l1
    f.restype = ctypes.c_double
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    loss = f(c.size // 3, c.ctypes.data, t.ctypes.data, G.ctypes.data)
    return loss, G


def ssim(x, y, radius=5, sigma=1.5, c1=1e-4, c2=9e-4, want_map=False, want_grad=False):
    """Mean SSIM of two [H][W][3] images (the reading in gs_oracle.c), optionally with the
    per-pixel map and d SSIM / d x.  Returns (ssim, map or None, grad or None)."""
    L = lib()
    a = _np(x, np.float32)
    b = _np(y, np.float32)
    assert a.shape == b.shape and a.ndim == 3 and a.shape[2] == 3
    H, W = a.shape[:2]
    smap = np.zeros(a.shape) if want_map else None
    grad = np.zeros(a.shape) if want_grad else None
    f = L.orc_ssim
    f.restype = ctypes.c_double
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                  ctypes.c_double, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
    val = f(W, H, a.ctypes.data, b.ctypes.data, radius, sigma, c1, c2,
            None if smap is None else smap.ctypes.data, None if grad is None else grad.ctypes.data)
    return val, smap, grad


def loss_l1_dssim(color, target, lam):
    """(1 - lam) L1 + lam (1 - SSIM) / 2 of two [H][W][3] images.  Returns (loss, G [H][W][3]
    float64 = dL/dcolor, ssim)."""
    L = lib()
    c = _np(color, np.float32)
    t = _np(target, np.float32)
    assert c.shape == t.shape and c.ndim == 3 and c.shape[2] == 3
    H, W = c.shape[:2]
    G = np.zeros(c.shape)
    s = ctypes.c_double(0.0)
    f = L.orc_loss_l1_dssim
    f.restype = ctypes.c_double
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                  ctypes.POINTER(ctypes.c_double)]
    loss = f(W, H, c.ctypes.data, t.ctypes.data, float(lam), G.ctypes.data, ctypes.byref(s))
    return loss, G, s.value


def adam(p, g, m, v, lr, b1, b2, eps, step):
    L = lib()
    p, g, m, v = (_np(x, np.float64).reshape(-1) for x in (p, g, m, v))
    n = p.size
    po, mo, vo = np.zeros(n), np.zeros(n), np.zeros(n)
    f = L.orc_adam
    f.restype = None
    f.argtypes = [ctypes.c_int64] + [ctypes.c_void_p] * 4 + [ctypes.c_double] * 4 + [ctypes.c_int] + [
        ctypes.c_void_p] * 3
    f(n, p.ctypes.data, g.ctypes.data, m.ctypes.data, v.ctypes.data, lr, b1, b2, eps, step,
      po.ctypes.data, mo.ctypes.data, vo.ctypes.data)
    return po, mo, vo


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def composite(cs, ts, t_min):
    L = lib()
    cs = [_np(c, np.float32).reshape(-1) for c in cs]
    ts = [_np(t, np.float32).reshape(-1) for t in ts]
    n_px = ts[0].size
    c_out, t_out = np.zeros(3 * n_px), np.zeros(n_px)
    f = L.orc_composite
    f.restype = None
    f.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                  ctypes.c_void_p, ctypes.c_void_p]
    f(len(cs), n_px, _ptr_array(cs), _ptr_array(ts), t_min, c_out.ctypes.data, t_out.ctypes.data)
    return c_out.reshape(n_px, 3), t_out


def composite_bwd(cs, ts, t_min, G, GT=None):
    L = lib()
    cs = [_np(c, np.float32).reshape(-1) for c in cs]
    ts = [_np(t, np.float32).reshape(-1) for t in ts]
    n_px = ts[0].size
    G = np.ascontiguousarray(np.asarray(G, np.float64).reshape(-1))
    gt_ptr = None
    if GT is not None:
        GT = np.ascontiguousarray(np.asarray(GT, np.float64).reshape(-1))
        gt_ptr = GT.ctypes.data
    dcs = [np.zeros(3 * n_px) for _ in cs]
    dts = [np.zeros(n_px) for _ in cs]
    f = L.orc_composite_bwd
    f.restype = None
    f.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f(len(cs), n_px, _ptr_array(cs), _ptr_array(ts), t_min, G.ctypes.data, gt_ptr, _ptr_array(dcs),
      _ptr_array(dts))
    return [d.reshape(n_px, 3) for d in dcs], dts


def compact(grads2d, index_base=0):
    """Returns (records [R][10] uint32, bitmap [ceil(n/32)] uint32)."""
    L = lib()
    g = _np(grads2d, np.float32)
    n = g.shape[1]
    rec = np.zeros((max(n, 1), 10), np.uint32)
    bm = np.zeros(max((n + 31) // 32, 1), np.uint32)
    f = L.orc_compact
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    R = f(n, g.ctypes.data, index_base, rec.ctypes.data, bm.ctypes.data)
    return rec[:R].copy(), bm[:(n + 31) // 32].copy()


def decode(parts, n_owner, out=None):
    """parts: list of (records [R][10] uint32, index_base, owner_index [n_part] or None,
    n_part).  Returns (grads [9][n_owner] float64 accumulated onto `out`, rejected)."""
    L = lib()
    k = len(parts)
    recs = [np.ascontiguousarray(np.asarray(p[0], np.uint32).reshape(-1, 10)) for p in parts]
    maps = [None if p[2] is None else np.ascontiguousarray(np.asarray(p[2], np.uint32)) for p in parts]
    res = np.zeros((9, n_owner)) if out is None else np.array(out, np.float64, copy=True).reshape(9, n_owner)
    res = np.ascontiguousarray(res)
    R = (ctypes.c_int64 * max(k, 1))(*[x.shape[0] for x in recs])
    base = (ctypes.c_uint32 * max(k, 1))(*[int(p[1]) for p in parts])
    npart = (ctypes.c_int64 * max(k, 1))(*[int(p[3]) for p in parts])
    rp = (ctypes.c_void_p * max(k, 1))(*[x.ctypes.data for x in recs])
    mp = (ctypes.c_void_p * max(k, 1))(*[None if m is None else m.ctypes.data for m in maps])
    f = L.orc_decode
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    rej = f(k, rp, R, base, mp, npart, n_owner, res.ctypes.data)
    return res, int(rej)


def adam_batch_hparams(bs, lrs, beta1=0.9, beta2=0.999, eps=1e-15):
    """(lrs [6], beta1, beta2, eps) scaled for BS views per step, or None if degenerate."""
    L = lib()
    lr = (ctypes.c_double * 6)(*[float(x) for x in lrs])
    b1, b2, e = ctypes.c_double(beta1), ctypes.c_double(beta2), ctypes.c_double(eps)
    f = L.orc_adam_batch_hparams
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    if f(int(bs), lr, ctypes.byref(b1), ctypes.byref(b2), ctypes.byref(e)) != 0:
        return None
    return list(lr), b1.value, b2.value, e.value


def sh_basis(deg, dirs):
    """Y [m][(deg+1)^2] and dY [m][(deg+1)^2][3] at unit vectors dirs [m][3]."""
    L = lib()
    d = np.ascontiguousarray(dirs, np.float64).reshape(-1, 3)
    K = (deg + 1) ** 2
    Y = np.zeros((d.shape[0], K))
    dY = np.zeros((d.shape[0], K, 3))
    f = L.orc_sh_basis
    f.restype = None
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for i in range(d.shape[0]):
        row = np.ascontiguousarray(d[i])
        y = np.zeros(K)
        g = np.zeros(3 * K)
        f(deg, row.ctypes.data, y.ctypes.data, g.ctypes.data)
        Y[i] = y
        dY[i] = g.reshape(K, 3)
    return Y, dY


def train_view(scene, cam, target, params: Params = Params(), with_grads3d=True):
    """Forward, L1 loss and backward of one view (full image). Returns a dict."""
    P = project(scene, cam, params)
    color, tf, nt, tie = render(P, params)
    loss, G = loss_l1(color.astype(np.float32), target)
    g2 = raster_backward(P, G.reshape(-1, 3), None, params)
    out = dict(proj=P, color=color, t_final=tf, n_trav=nt, tie=tie, loss=loss, G=G, grads2d=g2)
    if with_grads3d:
        out["grads3d"] = project_backward(scene, cam, g2, params)
    return out


def quat_to_rot(q):
    L = lib()
    qq = np.ascontiguousarray(q, np.float64).reshape(4)
    R = np.zeros(9)
    f = L.orc_quat_to_rot
    f.restype = None
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    f(qq.ctypes.data, R.ctypes.data)
    return R.reshape(3, 3)
