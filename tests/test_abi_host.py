"""Host-side checks of the C ABI and the Python layers (no GPU needed).

The library must load and export every function include/gs.h declares; argument
errors must be reported before anything is launched; workspace sizes and the
memory planner must follow their stated formulas.
"""
import ctypes
import json
import math
import os
import re

import numpy as np
import pytest

from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import memory, scenes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared():
    text = open(os.path.join(ROOT, "include", "gs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert len(declared) >= 14
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTED)


def test_struct_layouts_match_header():
    # sizes of the by-value structs the header defines (x86-64 SysV layout)
    assert ctypes.sizeof(B.Camera) == 16 * 4 + 4 * 4 + 2 * 4 + 4
    assert ctypes.sizeof(B.RasterParams) == 24
    assert ctypes.sizeof(B.Gaussians) == 5 * 8 + 8 + 8
    assert B.Gaussians.ld.offset == 48
    assert ctypes.sizeof(B.ParamGrads) == 5 * 8 + 8
    assert ctypes.sizeof(B.Projected) == 6 * 8
    assert ctypes.sizeof(B.Bins) == 4 * 8 + 8 + 8
    assert ctypes.sizeof(B.AdamGroup) == 4 * 8 + 8 + 8
    assert ctypes.sizeof(B.GradRecords) == 8 + 8 + 8 + 8 + 8      # uint32 index_base padded to 8
    assert B.GradRecords.owner_index.offset == 24


def _cam(w=64, h=48):
    return B.make_camera([1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 3, 0, 0, 0, 1], 50.0, 50.0, w / 2, h / 2, w, h)


def test_argument_errors_before_launch():
    g = B.Gaussians(None, None, None, None, None, 10)
    out = B.Projected(None, None, None, None, None, None)
    with pytest.raises(B.GsError) as e:
        B.gs_project(g, _cam(), B.make_params(0), out, stream=_NullStream())
    assert e.value.status == B.GS_ERR_INVALID_ARGUMENT and "NULL" in str(e.value)
    with pytest.raises(B.GsError) as e:
        B.gs_project(B.Gaussians(None, None, None, None, None, 0), _cam(), B.make_params(4), out, _NullStream())
    assert e.value.status == B.GS_ERR_UNSUPPORTED
    with pytest.raises(B.GsError) as e:
        B.gs_project(B.Gaussians(None, None, None, None, None, -1), _cam(), B.make_params(0), out, _NullStream())
    assert e.value.status == B.GS_ERR_INVALID_ARGUMENT
    with pytest.raises(B.GsError):
        B.gs_project(B.Gaussians(None, None, None, None, None, 0), _cam(0, 10), B.make_params(0), out, _NullStream())
    with pytest.raises(B.GsError):
        B.gs_project(B.Gaussians(None, None, None, None, None, 0), _cam(), B.make_params(0, alpha_max=1.0), out,
                     _NullStream())
    with pytest.raises(B.GsError):
        B.gs_project(B.Gaussians(None, None, None, None, None, 0), _cam(), B.make_params(0, t_min=2.0), out,
                     _NullStream())
    # Adam: too many groups, bad step
    st = B._lib.gs_adam_step(None, 17, 1, 0.9, 0.999, 1e-15, None)
    assert st == B.GS_ERR_INVALID_ARGUMENT
    st = B._lib.gs_adam_step(None, 0, 0, 0.9, 0.999, 1e-15, None)
    assert st == B.GS_ERR_INVALID_ARGUMENT
    # compositing: k out of range
    st = B._lib.gs_composite_over(None, None, 0, 10, 1e-4, None, None, None)
    assert st == B.GS_ERR_INVALID_ARGUMENT and "k must" in B.last_error()


def test_dssim_argument_errors_before_launch():
    """gs_loss_l1_dssim rejects sizes, NULL buffers, lambda outside [0, 1], images whose
    12 W H bytes need more than 32-bit offsets and short workspaces before any launch (the
    non-NULL addresses below are never dereferenced)."""
    fake = ctypes.c_void_p(256)
    call = lambda w, h, lam, ws_bytes, color=fake: B._lib.gs_loss_l1_dssim(
        color, fake, w, h, lam, None, None, fake, fake, ws_bytes, None)
    assert call(0, 10, 0.2, 1 << 30) == B.GS_ERR_INVALID_ARGUMENT
    assert call(70000, 10, 0.2, 1 << 30) == B.GS_ERR_INVALID_ARGUMENT
    assert call(16, 16, 0.2, 1 << 30, color=None) == B.GS_ERR_INVALID_ARGUMENT
    assert call(16, 16, 1.5, 1 << 30) == B.GS_ERR_INVALID_ARGUMENT
    assert call(16, 16, float("nan"), 1 << 30) == B.GS_ERR_INVALID_ARGUMENT
    assert call(20000, 20000, 0.2, 1 << 62) == B.GS_ERR_UNSUPPORTED and "2^32" in B.last_error()
    assert B.gs_loss_l1_dssim_workspace_bytes(20000, 20000) == 0
    assert B.gs_loss_l1_dssim_workspace_bytes(16384, 16384) >= 36 * 16384 * 16384
    assert call(16, 16, 0.2, B.gs_loss_l1_dssim_workspace_bytes(16, 16) - 1) == B.GS_ERR_INVALID_ARGUMENT


class _NullStream:
    cuda_stream = 0


def test_empty_inputs_return_ok_without_launch():
    out = B.Projected(None, None, None, None, None, None)
    B.gs_project(B.Gaussians(None, None, None, None, None, 0), _cam(), B.make_params(3), out, _NullStream())
    assert B._lib.gs_adam_step(None, 0, 1, 0.9, 0.999, 1e-15, None) == B.GS_OK


def test_workspace_sizes():
    a = B.gs_bin_sort_workspace_bytes(1000, 5000, 64, 64)
    b = B.gs_bin_sort_workspace_bytes(2000, 5000, 64, 64)
    c = B.gs_bin_sort_workspace_bytes(1000, 50000, 64, 64)
    assert 0 < a < b and a < c
    # O(32 B per Gaussian + 24 B per entry: two key and two value buffers for the tile
    # sort, the Gaussian and the first gradient slot of each emitted entry) plus histograms
    assert 24 * 45000 <= c - a < 24 * 45000 * 1.2 + 4 * 256 * 16 + 4096
    assert B.gs_bin_sort_workspace_bytes(-1, 0, 1, 1) == 0
    assert B.gs_compact_workspace_bytes(10**6) >= 4 * (10**6 // 256)
    assert B.gs_loss_workspace_bytes(100) >= 8
    # raster-ready lists: per entry 2 quadrant entries (Gaussian and slot, 8 B; tile-list
    # index, 4 B), gradient slots (36 B) and slot stamps (4 B); 4 quadrant bits and 4 prefix
    # counts per 64 entries; the first gradient slot and the raster record (64-B stride) per
    # Gaussian (+ the total); the raster order of the 4 quadrant waves per tile
    r0 = B.gs_bins_raster_bytes(5000, 64 * 1000, 1920, 1080)
    lo = 2 * (8 + 4 + 36 + 4) * 64000 + 4 * 8 * 1000 + 4 * 4 * 1001 + 4 * 5001 + 64 * 5000 + 4 * 4 * 8160
    assert lo <= r0 <= lo + 8 * 256
    assert B.gs_bins_raster_bytes(0, 0, 16, 16) > 0 and B.gs_bins_raster_bytes(0, -1, 16, 16) == 0


def test_memory_planner_matches_page_figures():
    """Per-Gaussian bytes of parameters + Adam moments and the resulting capacity of a
    192 GB accelerator, as printed on the ROCm blog page (golden fixture)."""
    gd = json.load(open(os.path.join(GOLDEN, "memory_per_gaussian.json")))
    assert memory.learnable_scalars(2) == gd["sh2"]["learnable_scalars"]
    assert 2 * memory.learnable_scalars(2) == gd["sh2"]["adam_scalars"]
    assert memory.bytes_per_gaussian(2) == gd["sh2"]["bytes_total"]
    assert memory.bytes_per_gaussian(2, adam=False) == gd["sh2"]["learnable_bytes"]
    assert memory.learnable_scalars(3) == gd["sh3"]["learnable_scalars"]
    assert memory.bytes_per_gaussian(3) == gd["sh3"]["bytes_total_approx"]
    hbm = gd["mi300x_hbm_bytes"]
    assert round(memory.max_gaussians(hbm, 3) / 1e6) == gd["gaussians_per_gpu_sh3_millions"]
    assert round(memory.max_gaussians(hbm, 2) / 1e6) == gd["gaussians_per_gpu_sh2_millions"]
    assert round(8 * memory.max_gaussians(hbm, 3) / 1e9, 2) == gd["gaussians_per_8gpu_node_sh3_billions"]
    # 1M Gaussians at SH2 -> 456 MB
    assert memory.bytes_per_gaussian(2) * 10**6 == 456 * 10**6
    # an MI355X holds the 20M-Gaussian workload's training state many times over
    assert memory.max_gaussians_training(memory.MI355X_HBM_BYTES, 3, 5.0) > 20 * 10**6


def test_scene_generators_are_seeded_and_shaped():
    a, b = scenes.scene_tiny(), scenes.scene_tiny()
    assert a.means.shape == (3, 1024) and a.sh.shape == (3, 1024)
    assert bool((a.means == b.means).all()) and bool((a.targets[0] == b.targets[0]).all())
    c = scenes.scene_100k()
    assert c.sh.shape == (48, 100_000) and c.cameras[0].width == 512
    assert abs(c.cameras[0].fx - 256 / math.tan(math.radians(30))) < 1e-9
    m2, r, d = scenes.projected_for_binning(1, 1000, 100, 50)
    assert (m2[:, 0] < 100).all() and (m2[:, 1] < 50).all() and (d > 0).all()


def test_tile_budget_and_fused_workspace():
    """ByteSplat Eq. 7: B = floor((M_budget - M_fixed) / M_g); -1 for arguments that do not
    define a budget.  The fused kernel's workspace holds one 16-byte partial per 8x8
    quadrant wave."""
    assert B.gs_tile_budget(65536, 10240, 48) == (65536 - 10240) // 48 == 1152
    assert B.gs_tile_budget(160 * 1024, 0, 48) == 3413
    assert B.gs_tile_budget(1000, 1000, 48) == 0
    assert B.gs_tile_budget(1000, 1001, 48) == -1
    assert B.gs_tile_budget(1000, 0, 0) == -1
    assert B.gs_tile_budget(-1, 0, 48) == -1
    # per-wave partials, the final reduction's per-block sums (one per 1024 waves) and its ticket
    waves = 120 * 68 * 4
    assert B.gs_raster_fused_l1_workspace_bytes(1920, 1080) == 16 * waves + 16 * -(-waves // 1024) + 16
    assert B.gs_raster_fused_l1_workspace_bytes(17, 1) == 16 * 8 + 16 + 16
    assert B.gs_raster_fused_l1_workspace_bytes(0, 10) == 0


def test_fused_l1_argument_errors_before_launch():
    g = B.Gaussians(None, None, None, None, None, 0)
    bins = B.Bins(None, None, None, None, 0, None)
    ws = _Buf(16)
    with pytest.raises(B.GsError) as e:   # no tile lists
        B._check(B._lib.gs_raster_fused_l1(ctypes.byref(g), ctypes.byref(bins), ctypes.byref(_cam()),
                                           ctypes.byref(B.make_params(0)), None, None, None, None, None, None,
                                           None, ws.ptr, 16, None))
    assert e.value.status == B.GS_ERR_INVALID_ARGUMENT
    with pytest.raises(B.GsError) as e:
        B._check(B._lib.gs_tile_budget_report(ctypes.byref(bins), ctypes.byref(_cam()), -1, None, None, None, None))
    assert e.value.status == B.GS_ERR_INVALID_ARGUMENT


def test_owner_update_argument_errors_before_launch():
    """gs_project_bwd_adam rejects a NULL gradient array, a step below 1, bad Adam
    hyper-parameters, NULL moments and a next camera without projection buffers before any
    launch, and returns OK without a launch when there are no Gaussians (the non-NULL
    addresses below are never dereferenced)."""
    fake = 256
    g = B.Gaussians(fake, fake, fake, fake, fake, 10)
    m = B.ParamGrads(fake, fake, fake, fake, fake)
    lr = B.AdamLrs(1e-3, 1e-3, 1e-3, 1e-3, 1e-3, 1e-3)
    p = B.make_params(3)
    empty = B.Projected(None, None, None, None, None, None)

    def call(gs=g, grads2d=fake, mm=m, step=1, b1=0.9, nc=None, np_=None):
        return B._lib.gs_project_bwd_adam(ctypes.byref(gs), ctypes.byref(_cam()), ctypes.byref(p), grads2d,
                                          ctypes.byref(mm) if mm is not None else None, ctypes.byref(m),
                                          ctypes.byref(lr), step, b1, 0.999, 1e-15,
                                          ctypes.byref(nc) if nc is not None else None,
                                          ctypes.byref(np_) if np_ is not None else None, None)
    assert call(grads2d=None) == B.GS_ERR_INVALID_ARGUMENT
    assert call(step=0) == B.GS_ERR_INVALID_ARGUMENT
    assert call(b1=1.0) == B.GS_ERR_INVALID_ARGUMENT
    assert call(mm=None) == B.GS_ERR_INVALID_ARGUMENT
    assert call(mm=B.ParamGrads(fake, None, fake, fake, fake)) == B.GS_ERR_INVALID_ARGUMENT
    assert call(nc=_cam()) == B.GS_ERR_INVALID_ARGUMENT
    assert call(nc=_cam(), np_=empty) == B.GS_ERR_INVALID_ARGUMENT
    assert call(gs=B.Gaussians(None, None, None, None, None, 0), grads2d=None) == B.GS_OK


def test_plane_stride_from_views_and_checks():
    """The binding takes the plane stride of [planes][n] views of padded [planes][ld]
    storage (0 for unpadded planes), rejects groups with different strides, and the library
    rejects a stride below n before any launch."""
    import torch
    store = torch.zeros(59, 128)
    v = store[:, :100]
    g = B.gaussians(v[0:3], v[3:6], v[6:10], v[10], v[11:])
    assert (g.n, g.ld) == (100, 128)
    pg = B.param_grads(v[0:3], v[3:6], v[6:10], v[10], v[11:])
    assert pg.ld == 128
    plain = torch.zeros(59, 100)
    assert B.gaussians(plain[0:3], plain[3:6], plain[6:10], plain[10], plain[11:]).ld == 0
    with pytest.raises(ValueError):
        B.gaussians(v[0:3], plain[3:6], v[6:10], v[10], v[11:])
    fake = 256
    bad = B.Gaussians(fake, fake, fake, fake, fake, 10, 8)
    out = B.Projected(fake, fake, fake, fake, fake, fake)
    with pytest.raises(B.GsError) as e:
        B.gs_project(bad, _cam(), B.make_params(3), out, _NullStream())
    assert e.value.status == B.GS_ERR_INVALID_ARGUMENT and "ld" in B.last_error()
    good = B.Gaussians(fake, fake, fake, fake, fake, 10, 64)
    m = B.ParamGrads(fake, fake, fake, fake, fake, 32)   # a moment stride other than the parameters'
    lr = B.AdamLrs(1e-3, 1e-3, 1e-3, 1e-3, 1e-3, 1e-3)
    st = B._lib.gs_project_bwd_adam(ctypes.byref(good), ctypes.byref(_cam()), ctypes.byref(B.make_params(3)), fake,
                                    ctypes.byref(m), ctypes.byref(m), ctypes.byref(lr), 1, 0.9, 0.999, 1e-15, None,
                                    None, None)
    assert st == B.GS_ERR_INVALID_ARGUMENT and "stride" in B.last_error()
    g3 = B.ParamGrads(fake, fake, fake, fake, fake, 5)
    assert B._lib.gs_project_bwd(ctypes.byref(good), ctypes.byref(_cam()), ctypes.byref(B.make_params(3)), fake,
                                 ctypes.byref(g3), None) == B.GS_ERR_INVALID_ARGUMENT


class _Buf:
    """A host buffer standing in for a device pointer in argument checks (never dereferenced)."""

    def __init__(self, n):
        self.mem = ctypes.create_string_buffer(n + 16)
        self.ptr = ctypes.c_void_p((ctypes.addressof(self.mem) + 15) // 16 * 16)


def test_decode_argument_errors_before_launch():
    """gs_decode_grads checks its partitions on the host; k = 0, empty partitions and an
    empty owner range with no counter launch nothing."""
    buf = _Buf(64)
    one = (B.GradRecords * 1)(B.GradRecords(buf.ptr, 1, 0, None, 1))
    st = B._lib.gs_decode_grads(one, 17, buf.ptr, 10, None, None)
    assert st == B.GS_ERR_INVALID_ARGUMENT and "k must" in B.last_error()
    assert B._lib.gs_decode_grads(None, 1, buf.ptr, 10, None, None) == B.GS_ERR_INVALID_ARGUMENT
    bad = (B.GradRecords * 1)(B.GradRecords(None, 5, 0, None, 10))
    assert B._lib.gs_decode_grads(bad, 1, buf.ptr, 10, None, None) == B.GS_ERR_INVALID_ARGUMENT
    neg = (B.GradRecords * 1)(B.GradRecords(buf.ptr, -1, 0, None, 10))
    assert B._lib.gs_decode_grads(neg, 1, buf.ptr, 10, None, None) == B.GS_ERR_INVALID_ARGUMENT
    odd = (B.GradRecords * 1)(B.GradRecords(ctypes.c_void_p(buf.ptr.value + 2), 1, 0, None, 1))
    assert B._lib.gs_decode_grads(odd, 1, buf.ptr, 10, None, None) == B.GS_ERR_INVALID_ARGUMENT
    assert B._lib.gs_decode_grads(one, 1, None, 10, None, None) == B.GS_ERR_INVALID_ARGUMENT
    assert B._lib.gs_decode_grads(one, 1, buf.ptr, -1, None, None) == B.GS_ERR_INVALID_ARGUMENT
    assert B._lib.gs_decode_grads(None, 0, None, 0, None, None) == B.GS_OK
    empty = (B.GradRecords * 1)(B.GradRecords(None, 0, 0, None, 0))
    assert B._lib.gs_decode_grads(empty, 1, None, 0, None, None) == B.GS_OK
    assert B._lib.gs_decode_grads(one, 1, None, 0, None, None) == B.GS_OK


def test_batch_hparams_match_oracle():
    """gs_adam_batch_hparams (host only) rounds the oracle's double-precision values once."""
    import oracle
    lrs = [1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3, 1.25e-4]
    lr = B.AdamLrs(*lrs)
    names = ("means", "log_scales", "quats", "opacity_logits", "sh_dc", "sh_rest")
    for bs in range(1, 11):
        out, b1, b2, e = B.gs_adam_batch_hparams(bs, lr)
        # the oracle scales the float32 rates the ABI receives
        o_lr, o_b1, o_b2, o_e = oracle.adam_batch_hparams(bs, [getattr(lr, nm) for nm in names])
        for nm, want in zip(names, o_lr):
            assert getattr(out, nm) == float(np.float32(want)), (bs, nm)
        assert b1 == float(np.float32(o_b1)) and b2 == float(np.float32(o_b2)) and e == float(np.float32(o_e))
    for bad in (0, 11):
        with pytest.raises(B.GsError):
            B.gs_adam_batch_hparams(bad, lr)


def test_batch_argument_errors_before_launch():
    g = B.Gaussians(None, None, None, None, None, 0)
    cams = (B.Camera * 5)(*([_cam()] * 5))
    outs = (B.Projected * 5)()
    p = B.make_params(3)
    assert B._lib.gs_project_batch(ctypes.byref(g), 0, cams, ctypes.byref(p), outs, None) == B.GS_ERR_INVALID_ARGUMENT
    assert B._lib.gs_project_batch(ctypes.byref(g), 5, cams, ctypes.byref(p), outs, None) == B.GS_ERR_INVALID_ARGUMENT
    assert B._lib.gs_project_batch(ctypes.byref(g), 2, cams, ctypes.byref(p), outs, None) == B.GS_OK   # n = 0
    bins = (B.Bins * 2)()
    m = B.ParamGrads()
    lr = B.AdamLrs()
    st = B._lib.gs_grad_aggregate_adam_batch(ctypes.byref(g), 2, bins, cams, ctypes.byref(p), 0.5, ctypes.byref(m),
                                             ctypes.byref(m), ctypes.byref(lr), 1, 0.9, 0.999, 1e-15, None, None, None)
    assert st == B.GS_ERR_INVALID_ARGUMENT      # the bins have no tile lists


def _signature(name):
    text = open(os.path.join(ROOT, "include", "gs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    return [" ".join(a.split()) for a in m.group(1).split(",")]


def _struct_fields(name):
    text = open(os.path.join(ROOT, "include", "gs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"typedef struct \{([^}]*)\}\s*" + name + r"\s*;", text)
    assert m, name
    return " ".join(m.group(1).split())


def test_boundary_departures_from_the_planned_abi_are_the_recorded_ones():
    """Where the C ABI differs from the planned boundary, it differs exactly as recorded:
    gs_bin_sort takes the raster parameters (alpha_min decides the quadrant lists);
    gs_raster_fwd reports the traversed entries per pixel (n_trav) and their sum instead of
    taking n_isect; gs_raster_bwd writes grads2d (no accumulation) and takes color and
    n_trav from the forward pass; gs_loss_l1 takes a workspace for its deterministic
    two-level sum; gs_adam_step reads the gradients without zeroing them; gs_projected holds
    the raster record, with the plain fields as optional planes and the radii interleaved;
    gs_bins holds the raster buffer, with keys and tiles_touched optional."""
    assert "const gs_raster_params *p" in _signature("gs_bin_sort")
    fwd = _signature("gs_raster_fwd")
    assert "int32_t *n_trav" in fwd and "unsigned long long *n_trav_sum" in fwd
    assert not any("n_isect" in a for a in fwd)
    bwd = _signature("gs_raster_bwd")
    assert "float *grads2d" in bwd and "const int32_t *n_trav" in bwd and "const float *color" in bwd
    loss = _signature("gs_loss_l1")
    assert "void *workspace" in loss and "size_t workspace_bytes" in loss
    adam = _signature("gs_adam_step")
    assert adam[0] == "const gs_adam_group *groups"
    assert "const float *g;" in _struct_fields("gs_adam_group")   # the gradients are an input only
    proj = _struct_fields("gs_projected")
    assert proj == "float *means2d, *conic_opacity, *color, *depth; int32_t *radii; float *rec;"
    bins = _struct_fields("gs_bins")
    assert "void *raster" in bins and "tiles_touched" in bins and "keys" in bins
    header = open(os.path.join(ROOT, "include", "gs.h")).read()
    assert "The gradients are read, not modified." in header
    assert "Every entry of\n * grads2d is written" in header
    assert "each pointer may be NULL,\n * and then that group is not written" in header
    # B9: the parameter, gradient and moment groups carry a plane stride
    assert _struct_fields("gs_gaussians").endswith("int64_t n; int64_t ld;")
    assert _struct_fields("gs_param_grads").endswith("int64_t ld;")
