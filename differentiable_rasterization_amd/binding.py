"""ctypes binding of libgsmi (include/gs.h).  Argument marshalling only.

Functions take torch tensors that live on the GPU and pass their device
pointers, with the current HIP stream, to the C ABI of the same name.  No
computation happens here; a non-OK status raises GsError with the library's
message.  torch is imported first so that the library binds to the HIP runtime
torch already loaded.  If libgsmi.so is missing the import fails loudly: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsmi.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m differentiable_rasterization_amd.build` "
                      "(or __graft_entry__.build()); there is no fallback implementation")

_lib = ctypes.CDLL(LIB_PATH)

GS_OK, GS_ERR_INVALID_ARGUMENT, GS_ERR_UNSUPPORTED, GS_ERR_CAPACITY, GS_ERR_HIP = range(5)
TILE = 16
EXPORTED = ("gs_project", "gs_bins_raster_bytes", "gs_bin_sort_workspace_bytes", "gs_bin_sort", "gs_bin_sort_async", "gs_raster_fwd", "gs_loss_workspace_bytes",
            "gs_loss_l1", "gs_loss_l1_dssim", "gs_loss_l1_dssim_workspace_bytes", "gs_raster_bwd", "gs_raster_bwd_partials", "gs_grad_aggregate", "gs_grad_aggregate_adam", "gs_grad_aggregate_adam_project",
            "gs_raster_fused_l1", "gs_raster_fused_l1_workspace_bytes", "gs_raster_fused_l1_noalloc",
            "gs_tile_budget", "gs_tile_budget_report",
            "gs_project_bwd", "gs_project_bwd_adam", "gs_adam_step", "gs_composite_over", "gs_composite_over_bwd",
            "gs_compact_workspace_bytes", "gs_compact_grads", "gs_decode_grads", "gs_project_batch",
            "gs_grad_aggregate_adam_batch", "gs_adam_batch_hparams", "gs_last_error")


class GsError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"gs status {status}: {message}")
        self.status = status


class GsCapacityError(GsError):
    def __init__(self, status, message, required):
        super().__init__(status, message)
        self.required = required


# ------------------------------------------------------------------ structs (mirror gs.h)

class Camera(ctypes.Structure):
    _fields_ = [("viewmat", ctypes.c_float * 16), ("fx", ctypes.c_float), ("fy", ctypes.c_float),
                ("cx", ctypes.c_float), ("cy", ctypes.c_float), ("width", ctypes.c_int32),
                ("height", ctypes.c_int32), ("near_z", ctypes.c_float)]


class RasterParams(ctypes.Structure):
    _fields_ = [("sh_degree", ctypes.c_int32), ("alpha_min", ctypes.c_float), ("alpha_max", ctypes.c_float),
                ("t_min", ctypes.c_float), ("depth_lo", ctypes.c_float), ("depth_hi", ctypes.c_float)]


class Gaussians(ctypes.Structure):
    _fields_ = [("means", ctypes.c_void_p), ("log_scales", ctypes.c_void_p), ("quats", ctypes.c_void_p),
                ("opacity_logits", ctypes.c_void_p), ("sh", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("ld", ctypes.c_int64)]


class Projected(ctypes.Structure):
    _fields_ = [("means2d", ctypes.c_void_p), ("conic_opacity", ctypes.c_void_p), ("color", ctypes.c_void_p),
                ("depth", ctypes.c_void_p), ("radii", ctypes.c_void_p), ("rec", ctypes.c_void_p)]


class Bins(ctypes.Structure):
    _fields_ = [("ids", ctypes.c_void_p), ("tile_ranges", ctypes.c_void_p), ("keys", ctypes.c_void_p),
                ("tiles_touched", ctypes.c_void_p), ("capacity", ctypes.c_int64), ("raster", ctypes.c_void_p)]


class ParamGrads(ctypes.Structure):
    _fields_ = [("means", ctypes.c_void_p), ("log_scales", ctypes.c_void_p), ("quats", ctypes.c_void_p),
                ("opacity_logits", ctypes.c_void_p), ("sh", ctypes.c_void_p), ("ld", ctypes.c_int64)]


class AdamLrs(ctypes.Structure):
    _fields_ = [(nm, ctypes.c_float) for nm in ("means", "log_scales", "quats", "opacity_logits", "sh_dc", "sh_rest")]


class AdamGroup(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("lr", ctypes.c_float)]


class GradRecords(ctypes.Structure):
    _fields_ = [("records", ctypes.c_void_p), ("r", ctypes.c_int64), ("index_base", ctypes.c_uint32),
                ("owner_index", ctypes.c_void_p), ("n_part", ctypes.c_int64)]


_P = ctypes.POINTER
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "gs_project": (_i32, [_P(Gaussians), _P(Camera), _P(RasterParams), _P(Projected), _vp]),
    "gs_bins_raster_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "gs_bin_sort_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "gs_bin_sort": (_i32, [_P(Projected), _i64, _P(Camera), _P(RasterParams), _P(Bins), _P(_i64), _vp, _sz, _vp]),
    "gs_bin_sort_async": (_i32, [_P(Projected), _i64, _P(Camera), _P(RasterParams), _P(Bins), _vp, _vp, _sz, _vp]),
    "gs_raster_fwd": (_i32, [_P(Projected), _P(Bins), _P(Camera), _P(RasterParams), _vp, _vp, _vp, _vp, _vp]),
    "gs_loss_workspace_bytes": (_sz, [_i64]),
    "gs_loss_l1": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "gs_loss_l1_dssim_workspace_bytes": (_sz, [_i32, _i32]),
    "gs_loss_l1_dssim": (_i32, [_vp, _vp, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gs_raster_bwd": (_i32, [_P(Gaussians), _P(Projected), _P(Bins), _P(Camera), _P(RasterParams), _vp, _vp, _vp,
                             _vp, _vp, _vp, _P(ParamGrads), _vp]),
    "gs_raster_bwd_partials": (_i32, [_P(Gaussians), _P(Bins), _P(Camera), _P(RasterParams), _vp, _vp, _vp, _vp,
                                      _vp, _vp]),
    "gs_grad_aggregate": (_i32, [_P(Gaussians), _P(Projected), _P(Bins), _P(Camera), _P(RasterParams), _vp,
                                 _P(ParamGrads), _vp]),
    "gs_grad_aggregate_adam": (_i32, [_P(Gaussians), _P(Projected), _P(Bins), _P(Camera), _P(RasterParams), _vp,
                                      _P(ParamGrads),
                                      _P(ParamGrads), _P(AdamLrs), _i32, _f32, _f32, _f32, _vp]),
    "gs_grad_aggregate_adam_project": (_i32, [_P(Gaussians), _P(Projected), _P(Bins), _P(Camera), _P(RasterParams),
                                              _vp, _P(ParamGrads), _P(ParamGrads), _P(AdamLrs), _i32, _f32, _f32,
                                              _f32, _P(Camera), _P(Projected), _vp]),
    "gs_project_bwd_adam": (_i32, [_P(Gaussians), _P(Camera), _P(RasterParams), _vp, _P(ParamGrads),
                                   _P(ParamGrads), _P(AdamLrs), _i32, _f32, _f32, _f32, _P(Camera), _P(Projected),
                                   _vp]),
    "gs_raster_fused_l1": (_i32, [_P(Gaussians), _P(Bins), _P(Camera), _P(RasterParams), _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "gs_raster_fused_l1_workspace_bytes": (ctypes.c_size_t, [_i32, _i32]),
    "gs_raster_fused_l1_noalloc": (_i32, [_P(Gaussians), _P(Bins), _P(Camera), _P(RasterParams), _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _vp]),
    "gs_tile_budget": (_i64, [_i64, _i64, _i64]),
    "gs_tile_budget_report": (_i32, [_P(Bins), _P(Camera), _i64, _vp, _vp, _vp, _vp]),
    "gs_project_bwd": (_i32, [_P(Gaussians), _P(Camera), _P(RasterParams), _vp, _P(ParamGrads), _vp]),
    "gs_adam_step": (_i32, [_P(AdamGroup), _i32, _i32, _f32, _f32, _f32, _vp]),
    "gs_composite_over": (_i32, [_P(_vp), _P(_vp), _i32, _i64, _f32, _vp, _vp, _vp]),
    "gs_composite_over_bwd": (_i32, [_P(_vp), _P(_vp), _i32, _i64, _f32, _vp, _vp, _P(_vp), _P(_vp), _vp]),
    "gs_compact_workspace_bytes": (_sz, [_i64]),
    "gs_compact_grads": (_i32, [_vp, _i64, ctypes.c_uint32, _vp, _vp, _P(_i64), _vp, _sz, _vp]),
    "gs_decode_grads": (_i32, [_P(GradRecords), _i32, _vp, _i64, _vp, _vp]),
    "gs_project_batch": (_i32, [_P(Gaussians), _i32, _P(Camera), _P(RasterParams), _P(Projected), _vp]),
    "gs_grad_aggregate_adam_batch": (_i32, [_P(Gaussians), _i32, _P(Bins), _P(Camera), _P(RasterParams), _f32,
                                            _P(ParamGrads), _P(ParamGrads), _P(AdamLrs), _i32, _f32, _f32, _f32,
                                            _P(Camera), _P(Projected), _vp]),
    "gs_adam_batch_hparams": (_i32, [_i32, ctypes.c_double, ctypes.c_double, ctypes.c_double, _P(AdamLrs),
                                     _P(AdamLrs), _P(_f32), _P(_f32), _P(_f32)]),
    "gs_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def last_error() -> str:
    return _lib.gs_last_error().decode()


def _check(status, required=None):
    if status != GS_OK:
        if status == GS_ERR_CAPACITY:
            raise GsCapacityError(status, last_error(), required)
        raise GsError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _plane_ptr(t):
    """The address of a [planes][n] parameter view whose rows are contiguous (the plane
    stride is checked by _plane_stride)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ argument builders

def make_camera(viewmat, fx, fy, cx, cy, width, height, near_z=0.01) -> Camera:
    vm = [float(x) for x in (viewmat.reshape(-1).tolist() if hasattr(viewmat, "reshape") else viewmat)]
    return Camera((ctypes.c_float * 16)(*vm), fx, fy, cx, cy, int(width), int(height), near_z)


def camera_from(cam) -> Camera:
    """From an object with viewmat, fx, fy, cx, cy, width, height (and near_z)."""
    return make_camera(cam.viewmat, cam.fx, cam.fy, cam.cx, cam.cy, cam.width, cam.height,
                       getattr(cam, "near_z", 0.01))


def make_params(sh_degree, alpha_min=1.0 / 255.0, alpha_max=0.99, t_min=1e-4, depth_lo=0.0,
                depth_hi=math.inf) -> RasterParams:
    return RasterParams(int(sh_degree), alpha_min, alpha_max, t_min, depth_lo, depth_hi)


def _plane_stride(groups, n):
    """The one plane stride of [planes][n] views (rows contiguous), 0 for plain [planes][n]."""
    ld = None
    for t in groups:
        if t.dim() == 2 and t.shape[0] > 1:
            if t.stride(1) != 1:
                raise ValueError("parameter planes must be contiguous rows")
            if ld is None:
                ld = t.stride(0)
            elif t.stride(0) != ld:
                raise ValueError("every parameter group must have the same plane stride")
        elif t.dim() >= 1 and t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("parameter planes must be contiguous rows")
    return 0 if ld is None or ld == n else ld


def gaussians(means, log_scales, quats, opacity_logits, sh) -> Gaussians:
    """[planes][n] tensors (views of [planes][ld] storage allowed: the plane stride is
    taken from them and must be the same for every group)."""
    n = means.shape[-1]
    ld = _plane_stride((means, log_scales, quats, opacity_logits, sh), n)
    return Gaussians(_plane_ptr(means), _plane_ptr(log_scales), _plane_ptr(quats), _plane_ptr(opacity_logits),
                     _plane_ptr(sh), n, ld)


def projected(means2d, conic_opacity, color, depth, radii, rec) -> Projected:
    return Projected(_ptr(means2d), _ptr(conic_opacity), _ptr(color), _ptr(depth), _ptr(radii), _ptr(rec))


def bins(ids, tile_ranges, raster, keys=None, tiles_touched=None) -> Bins:
    """ids [capacity] int32/uint32, tile_ranges [tiles+1] int32, raster: a uint8 device buffer of
    gs_bins_raster_bytes(n, capacity, W, H) bytes."""
    return Bins(_ptr(ids), _ptr(tile_ranges), _ptr(keys), _ptr(tiles_touched), ids.numel(), _ptr(raster))


def param_grads(means, log_scales, quats, opacity_logits, sh) -> ParamGrads:
    n = means.shape[-1]
    ld = _plane_stride((means, log_scales, quats, opacity_logits, sh), n)
    return ParamGrads(_plane_ptr(means), _plane_ptr(log_scales), _plane_ptr(quats), _plane_ptr(opacity_logits),
                      _plane_ptr(sh), ld)


# ------------------------------------------------------------------ entry points (same names as the C ABI)

def gs_project(g: Gaussians, cam: Camera, p: RasterParams, out: Projected, stream=None):
    _check(_lib.gs_project(ctypes.byref(g), ctypes.byref(cam), ctypes.byref(p), ctypes.byref(out), _stream(stream)))


def gs_bins_raster_bytes(n, capacity, width, height) -> int:
    return int(_lib.gs_bins_raster_bytes(n, capacity, width, height))


def gs_bin_sort_workspace_bytes(n, capacity, width, height) -> int:
    return int(_lib.gs_bin_sort_workspace_bytes(n, capacity, width, height))


def gs_bin_sort(proj: Projected, n, cam: Camera, p: RasterParams, b: Bins, workspace, stream=None) -> int:
    """Returns K.  Raises GsCapacityError (with .required = the capacity needed) if the lists
    are too small."""
    k = _i64(0)
    st = _lib.gs_bin_sort(ctypes.byref(proj), n, ctypes.byref(cam), ctypes.byref(p), ctypes.byref(b), ctypes.byref(k),
                          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, required=k.value)
    return k.value


def gs_bin_sort_async(proj: Projected, n, cam: Camera, p: RasterParams, b: Bins, counts, workspace, stream=None):
    """Queues the sort without waiting for the device; counts (device int64[2], or None)
    receives (K, required capacity or 0)."""
    _check(_lib.gs_bin_sort_async(ctypes.byref(proj), n, ctypes.byref(cam), ctypes.byref(p), ctypes.byref(b),
                                  _ptr(counts), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))


def gs_raster_fwd(proj: Projected, b: Bins, cam: Camera, p: RasterParams, color, t_final, n_trav, n_trav_sum=None,
                  stream=None):
    _check(_lib.gs_raster_fwd(ctypes.byref(proj), ctypes.byref(b), ctypes.byref(cam), ctypes.byref(p), _ptr(color),
                              _ptr(t_final), _ptr(n_trav), _ptr(n_trav_sum), _stream(stream)))


def gs_loss_workspace_bytes(n_px) -> int:
    return int(_lib.gs_loss_workspace_bytes(n_px))


def gs_loss_l1(color, target, n_px, loss_out, dL_dcolor, workspace, stream=None):
    _check(_lib.gs_loss_l1(_ptr(color), _ptr(target), n_px, _ptr(loss_out), _ptr(dL_dcolor), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))


def gs_raster_bwd(g: Gaussians, proj: Projected, b: Bins, cam: Camera, p: RasterParams, color, t_final, n_trav,
                  dL_dcolor, dL_dt, grads2d, grads3d: ParamGrads | None, stream=None):
    _check(_lib.gs_raster_bwd(ctypes.byref(g), ctypes.byref(proj), ctypes.byref(b), ctypes.byref(cam),
                              ctypes.byref(p), _ptr(color), _ptr(t_final), _ptr(n_trav), _ptr(dL_dcolor), _ptr(dL_dt),
                              _ptr(grads2d), ctypes.byref(grads3d) if grads3d is not None else None,
                              _stream(stream)))


def gs_raster_bwd_partials(g: Gaussians, b: Bins, cam: Camera, p: RasterParams, color, t_final, n_trav, dL_dcolor,
                           dL_dt, stream=None):
    _check(_lib.gs_raster_bwd_partials(ctypes.byref(g), ctypes.byref(b), ctypes.byref(cam), ctypes.byref(p),
                                       _ptr(color), _ptr(t_final), _ptr(n_trav), _ptr(dL_dcolor), _ptr(dL_dt),
                                       _stream(stream)))


def gs_grad_aggregate(g: Gaussians, proj: Projected, b: Bins, cam: Camera, p: RasterParams, grads2d,
                      grads3d: ParamGrads | None, stream=None):
    _check(_lib.gs_grad_aggregate(ctypes.byref(g), ctypes.byref(proj), ctypes.byref(b), ctypes.byref(cam), ctypes.byref(p),
                                  _ptr(grads2d), ctypes.byref(grads3d) if grads3d is not None else None,
                                  _stream(stream)))


def gs_grad_aggregate_adam(g: Gaussians, proj: Projected, b: Bins, cam: Camera, p: RasterParams, grads2d,
                           m: ParamGrads, v: ParamGrads, lr: "AdamLrs", step, beta1, beta2, eps, stream=None):
    _check(_lib.gs_grad_aggregate_adam(ctypes.byref(g), ctypes.byref(proj), ctypes.byref(b), ctypes.byref(cam),
                                       ctypes.byref(p),
                                       _ptr(grads2d), ctypes.byref(m), ctypes.byref(v), ctypes.byref(lr), step, beta1,
                                       beta2, eps, _stream(stream)))


def gs_grad_aggregate_adam_project(g: Gaussians, proj: Projected, b: Bins, cam: Camera, p: RasterParams, grads2d,
                                   m: ParamGrads, v: ParamGrads, lr: "AdamLrs", step, beta1, beta2, eps,
                                   next_cam: Camera, next_proj: Projected, stream=None):
    _check(_lib.gs_grad_aggregate_adam_project(ctypes.byref(g), ctypes.byref(proj), ctypes.byref(b),
                                               ctypes.byref(cam), ctypes.byref(p), _ptr(grads2d), ctypes.byref(m),
                                               ctypes.byref(v), ctypes.byref(lr), step, beta1, beta2, eps,
                                               ctypes.byref(next_cam), ctypes.byref(next_proj), _stream(stream)))


def gs_project_bwd_adam(g: Gaussians, cam: Camera, p: RasterParams, grads2d, m: ParamGrads, v: ParamGrads,
                        lr: "AdamLrs", step, beta1, beta2, eps, next_cam: Camera = None, next_proj: Projected = None,
                        stream=None):
    _check(_lib.gs_project_bwd_adam(ctypes.byref(g), ctypes.byref(cam), ctypes.byref(p), _ptr(grads2d),
                                    ctypes.byref(m), ctypes.byref(v), ctypes.byref(lr), step, beta1, beta2, eps,
                                    ctypes.byref(next_cam) if next_cam is not None else None,
                                    ctypes.byref(next_proj) if next_proj is not None else None, _stream(stream)))


def gs_loss_l1_dssim_workspace_bytes(width, height) -> int:
    return int(_lib.gs_loss_l1_dssim_workspace_bytes(width, height))


def gs_loss_l1_dssim(color, target, width, height, lam, loss_out, ssim_out, dL_dcolor, workspace, stream=None):
    _check(_lib.gs_loss_l1_dssim(_ptr(color), _ptr(target), int(width), int(height), float(lam), _ptr(loss_out),
                                 _ptr(ssim_out), _ptr(dL_dcolor), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def gs_raster_fused_l1_workspace_bytes(width, height) -> int:
    return int(_lib.gs_raster_fused_l1_workspace_bytes(width, height))


def gs_raster_fused_l1(g: Gaussians, b: Bins, cam: Camera, p: RasterParams, target, color, t_final, n_trav,
                       loss_out, n_trav_sum, workspace, stream=None, walk_counts=None):
    _check(_lib.gs_raster_fused_l1(ctypes.byref(g), ctypes.byref(b), ctypes.byref(cam), ctypes.byref(p), _ptr(target),
                                   _ptr(color), _ptr(t_final), _ptr(n_trav), _ptr(loss_out), _ptr(n_trav_sum),
                                   _ptr(walk_counts), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


FUSED_NOALLOC_MAX_WAVES = 256 * 256 * 4


def gs_raster_fused_l1_noalloc(g: Gaussians, b: Bins, cam: Camera, p: RasterParams, target, color, t_final, n_trav,
                               loss_out, n_trav_sum, stream=None, walk_counts=None):
    _check(_lib.gs_raster_fused_l1_noalloc(ctypes.byref(g), ctypes.byref(b), ctypes.byref(cam), ctypes.byref(p),
                                           _ptr(target), _ptr(color), _ptr(t_final), _ptr(n_trav), _ptr(loss_out),
                                           _ptr(n_trav_sum), _ptr(walk_counts), _stream(stream)))


def gs_tile_budget(lds_budget_bytes, fixed_bytes, bytes_per_gaussian) -> int:
    return int(_lib.gs_tile_budget(lds_budget_bytes, fixed_bytes, bytes_per_gaussian))


def gs_tile_budget_report(b: Bins, cam: Camera, budget, excess=None, frac=None, totals=None, stream=None):
    _check(_lib.gs_tile_budget_report(ctypes.byref(b), ctypes.byref(cam), budget, _ptr(excess), _ptr(frac),
                                      _ptr(totals), _stream(stream)))


def gs_project_bwd(g: Gaussians, cam: Camera, p: RasterParams, grads2d, grads3d: ParamGrads, stream=None):
    _check(_lib.gs_project_bwd(ctypes.byref(g), ctypes.byref(cam), ctypes.byref(p), _ptr(grads2d),
                               ctypes.byref(grads3d), _stream(stream)))


def gs_adam_step(groups, step, beta1=0.9, beta2=0.999, eps=1e-15, stream=None):
    """groups: list of (p, g, m, v, lr) tensors / floats."""
    arr = (AdamGroup * max(len(groups), 1))()
    for i, (p, g, m, v, lr) in enumerate(groups):
        arr[i] = AdamGroup(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.numel(), lr)
    _check(_lib.gs_adam_step(arr, len(groups), int(step), beta1, beta2, eps, _stream(stream)))


def _ptr_list(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def gs_composite_over(c_k, t_k, n_px, t_min, c_out, t_out, stream=None):
    _check(_lib.gs_composite_over(_ptr_list(c_k), _ptr_list(t_k), len(c_k), n_px, t_min, _ptr(c_out), _ptr(t_out),
                                  _stream(stream)))


def gs_composite_over_bwd(c_k, t_k, n_px, t_min, dL_dc, dL_dt, dL_dc_k, dL_dt_k, stream=None):
    _check(_lib.gs_composite_over_bwd(_ptr_list(c_k), _ptr_list(t_k), len(c_k), n_px, t_min, _ptr(dL_dc),
                                      _ptr(dL_dt), _ptr_list(dL_dc_k), _ptr_list(dL_dt_k), _stream(stream)))


def gs_compact_workspace_bytes(n) -> int:
    return int(_lib.gs_compact_workspace_bytes(n))


def gs_compact_grads(grads2d, n, index_base, records, bitmap, workspace, stream=None) -> int:
    r = _i64(0)
    _check(_lib.gs_compact_grads(_ptr(grads2d), n, index_base, _ptr(records), _ptr(bitmap), ctypes.byref(r),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return r.value


def gs_decode_grads(parts, grads2d, n_owner, rejected=None, stream=None):
    """parts: list of (records, r, index_base, owner_index or None, n_part); adds the
    records' fields into grads2d [9][n_owner]."""
    arr = (GradRecords * max(len(parts), 1))()
    for i, (rec, r, base, owner, n_part) in enumerate(parts):
        arr[i] = GradRecords(_ptr(rec), int(r), int(base), _ptr(owner), int(n_part))
    _check(_lib.gs_decode_grads(arr, len(parts), _ptr(grads2d), int(n_owner), _ptr(rejected), _stream(stream)))


def _array(cls, items):
    arr = (cls * len(items))()
    for k, it in enumerate(items):
        arr[k] = it
    return arr


def gs_project_batch(g: Gaussians, cams, p: RasterParams, outs, stream=None):
    """cams: list of Camera; outs: list of Projected (one per camera)."""
    _check(_lib.gs_project_batch(ctypes.byref(g), len(cams), _array(Camera, cams), ctypes.byref(p),
                                 _array(Projected, outs), _stream(stream)))


def gs_grad_aggregate_adam_batch(g: Gaussians, bins, cams, p: RasterParams, grad_scale, m: ParamGrads,
                                 v: ParamGrads, lr: "AdamLrs", step, beta1, beta2, eps, next_cams=None,
                                 next_projs=None, stream=None):
    """bins, cams: lists (one per view); next_cams / next_projs: lists or None."""
    nc = _array(Camera, next_cams) if next_cams is not None else None
    npj = _array(Projected, next_projs) if next_projs is not None else None
    _check(_lib.gs_grad_aggregate_adam_batch(ctypes.byref(g), len(cams), _array(Bins, bins), _array(Camera, cams),
                                             ctypes.byref(p), grad_scale, ctypes.byref(m), ctypes.byref(v),
                                             ctypes.byref(lr), int(step), beta1, beta2, eps, nc, npj, _stream(stream)))


def gs_adam_batch_hparams(batch, lr: "AdamLrs", beta1=0.9, beta2=0.999, eps=1e-15):
    """(learning rates, beta1, beta2, eps) for a batch of `batch` views."""
    out = AdamLrs()
    b1, b2, e = _f32(), _f32(), _f32()
    _check(_lib.gs_adam_batch_hparams(int(batch), beta1, beta2, eps, ctypes.byref(lr), ctypes.byref(out),
                                      ctypes.byref(b1), ctypes.byref(b2), ctypes.byref(e)))
    return out, b1.value, b2.value, e.value
