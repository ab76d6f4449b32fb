"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded
synthetic inputs.  GPU only.

Tolerances: projected records within a few float32 ulps (both sides project in
double and round once); binning and compaction bit-exact; images and final
transmittance within 1e-4 max |difference| outside tie pixels; screen-space and
parameter gradients within relative L2 error 1e-3 per tensor (float32 atomics);
Adam within 1e-6 relative per tensor.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import pipeline as PL
from differentiable_rasterization_amd import scenes
from tests.gpu_util import (DEV, compare_images, compare_projection, gpu_forward, log, oracle_params, rel_l2,
                            synthetic_projection, ulp_diff)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": lambda: scenes.scene_tiny(),
    "ragged_sh1": lambda: scenes.scene_small_random(11, 600, 77, 53, 1, extent=1.2, distance=3.0),
    "ragged_sh2": lambda: scenes.scene_small_random(12, 3000, 130, 33, 2, extent=1.5, distance=3.0,
                                                    log_scale_mean=-3.0),
    "offscreen_sh3": lambda: scenes.scene_small_random(13, 2000, 96, 80, 3, extent=4.0, distance=3.0,
                                                       log_scale_mean=-2.5, logit_mean=1.0),
}


def _scene(name):
    if name == "100k":
        return scenes.scene_100k()
    return SMALL[name]()


# ------------------------------------------------------------------ projection

@pytest.mark.parametrize("name", ["tiny", "ragged_sh1", "ragged_sh2", "offscreen_sh3", "100k"])
def test_project_parity(name):
    log(f"project parity {name}")
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    st = gpu_forward(sc, cam, rp)
    P = oracle.project(sc, cam, oracle_params(rp))
    stats = compare_projection(st.proj, P)
    assert 0 < stats["visible"] <= sc.n
    log(f"  {stats}")


def test_project_culls_nonfinite_and_window():
    sc = scenes.scene_small_random(14, 256, 64, 48, 1, extent=1.0)
    sc.means[0, 3] = float("nan")
    sc.log_scales[1, 5] = float("inf")
    sc.quats[:, 7] = 0.0
    sc.sh[2, 9] = float("nan")
    cam = sc.cameras[0]
    lo, hi = float(np.float32(2.7)), float(np.float32(3.3))
    rp = B.make_params(1, depth_lo=lo, depth_hi=hi)
    st = gpu_forward(sc, cam, rp)
    P = oracle.project(sc, cam, oracle_params(rp))
    radii = st.proj.radii.cpu().numpy()
    vis_g = (radii[:, 0] > 0)
    for i in (3, 5, 7, 9):
        assert not vis_g[i]
    assert np.array_equal(vis_g, P.vis.astype(bool))
    dk = st.proj.depth.cpu().numpy()
    assert np.all((dk[vis_g] >= lo) & (dk[vis_g] < hi))


# ------------------------------------------------------------------ binning (bit-exact)

def _bin_gpu(m2, r, d, W, H, capacity=None):
    n = d.numel()
    cam = B.make_camera([1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1], 1.0, 1.0, 0.0, 0.0, W, H)
    proj = synthetic_projection(m2, r, d)
    bins = PL.Binning(n, W, H, capacity=capacity or 0, device=DEV, with_keys=True, with_touched=True)
    k = bins.sort(proj, cam, B.make_params(0))
    torch.cuda.synchronize()
    return k, bins


@pytest.mark.parametrize("n,W,H,maxr,seed", [
    (0, 64, 64, 8, 1), (1, 64, 64, 8, 2), (7, 16, 16, 3, 3), (3000, 100, 70, 30, 4), (20000, 257, 129, 60, 5),
    (200000, 1920, 1080, 24, 6), (50000, 3840, 2160, 300, 7), (5000, 4096, 4096, 2000, 8),
])
def test_bin_sort_bit_exact(n, W, H, maxr, seed):
    log(f"bin sort n={n} {W}x{H}")
    m2, r, d = scenes.projected_for_binning(seed, n, W, H, max_radius=maxr)
    k, bins = _bin_gpu(m2, r, d, W, H)
    tt, keys, ids, ranges = oracle.bin_f32(m2, r, d, W, H)
    assert k == len(ids)
    assert np.array_equal(bins.tile_ranges.cpu().numpy(), ranges)
    if n:
        assert np.array_equal(bins.tiles_touched.cpu().numpy(), tt)
    if k:
        assert np.array_equal(bins.ids[:k].cpu().numpy().view(np.uint32), ids)
        assert np.array_equal(bins.keys[:k].cpu().numpy().view(np.uint64), keys)


@pytest.mark.parametrize("n,span,seed", [
    (2, 0, 11), (3000, 0, 12), (20000, 0xFFFFFE, 13), (20000, 0xFFFFFF, 14), (20000, 0x1000000, 15),
    (200000, 0x7FFFFF, 16),
])
def test_bin_sort_depth_key_span(n, span, seed):
    """The depth sort orders by the float bits of the depth; visible depths whose keys span
    at most 2^24 - 2 take a shorter path than wider ones.  Depths here are built from their
    bit patterns at the edges of that range (the smallest and the largest key both present,
    repeated keys included); the lists must equal the oracle's either way."""
    log(f"bin sort depth key span n={n} span={span:#x}")
    W, H = 640, 360
    m2, r, _ = scenes.projected_for_binning(seed, n, W, H, max_radius=20)
    g = np.random.default_rng(seed)
    base = np.uint32(np.float32(20.0).view(np.uint32))
    off = g.integers(0, span + 1, size=n, dtype=np.int64)
    off[g.random(n) < 0.1] = span // 3
    vis = np.flatnonzero((r[:, 0] > 0).numpy())
    if len(vis) >= 2:
        off[vis[0]], off[vis[-1]] = span, 0
    d = torch.from_numpy((base + off.astype(np.uint32)).view(np.float32).copy())
    k, bins = _bin_gpu(m2, r, d, W, H)
    tt, keys, ids, ranges = oracle.bin_f32(m2, r, d, W, H)
    assert k == len(ids)
    assert np.array_equal(bins.tile_ranges.cpu().numpy(), ranges)
    assert np.array_equal(bins.tiles_touched.cpu().numpy(), tt)
    if k:
        assert np.array_equal(bins.ids[:k].cpu().numpy().view(np.uint32), ids)
        assert np.array_equal(bins.keys[:k].cpu().numpy().view(np.uint64), keys)


def test_bin_sort_all_culled_and_capacity():
    m2, r, d = scenes.projected_for_binning(9, 4000, 200, 150, max_radius=20)
    r0 = torch.zeros_like(r)
    k, bins = _bin_gpu(m2, r0, d, 200, 150)
    assert k == 0 and int(bins.tile_ranges.abs().sum()) == 0
    # capacity error reports the required size and leaves the caller to grow
    tt, keys, ids, ranges = oracle.bin_f32(m2, r, d, 200, 150)
    cam = B.make_camera([1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1], 1.0, 1.0, 0.0, 0.0, 200, 150)
    proj = synthetic_projection(m2, r, d)
    small = PL.Binning(4000, 200, 150, capacity=10, device=DEV)
    with pytest.raises(B.GsCapacityError) as ei:
        B.gs_bin_sort(proj.abi(), 4000, cam, B.make_params(0), small.abi(), small.workspace)
    # the required capacity is max(K, ceil(Q / 2)); with a zero conic every entry reaches all
    # four quadrants of its tile, so Q = 4 K
    assert ei.value.required == 2 * len(ids)


def test_bin_sort_async_matches_sync_and_reports_overflow():
    """gs_bin_sort_async gives gs_bin_sort's lists and image bit for bit; when the lists do
    not fit it reports the required capacity in its device counts and leaves every tile
    list empty (nothing rendered, zero gradients)."""
    sc = SMALL["ragged_sh2"]()
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    st = gpu_forward(sc, cam, rp)
    c = B.camera_from(cam)
    k_sync = st.bins.n_isect
    ids0, rng0 = st.bins.ids[:k_sync].clone(), st.bins.tile_ranges.clone()
    col0, t0, n0 = st.frame.color.clone(), st.frame.t_final.clone(), st.frame.n_trav.clone()
    counts = torch.full((2,), -7, dtype=torch.int64, device=DEV)
    st.bins.ids.zero_(); st.bins.tile_ranges.fill_(-1)
    st.bins.sort_async(st.proj, c, rp, counts)
    f = st.frame
    B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), c, rp, f.color, f.t_final, f.n_trav)
    torch.cuda.synchronize()
    assert counts.tolist() == [k_sync, 0]
    assert torch.equal(st.bins.ids[:k_sync], ids0) and torch.equal(st.bins.tile_ranges, rng0)
    assert torch.equal(f.color, col0) and torch.equal(f.t_final, t0) and torch.equal(f.n_trav, n0)
    # too small: the sync call's error and the async call's counts agree
    n = sc.n
    small = PL.Binning(n, cam.width, cam.height, capacity=16, device=DEV)
    with pytest.raises(B.GsCapacityError) as ei:
        B.gs_bin_sort(st.proj.abi(), n, c, rp, small.abi(), small.workspace)
    small.sort_async(st.proj, c, rp, counts)
    B.gs_raster_fwd(st.proj.abi(), small.abi(), c, rp, f.color, f.t_final, f.n_trav)
    g2 = torch.full((9, n), float("nan"), device=DEV)
    B.gs_raster_bwd(st.params.gaussians(), st.proj.abi(), small.abi(), c, rp, f.color, f.t_final, f.n_trav,
                    torch.ones_like(f.color), None, g2, None)
    torch.cuda.synchronize()
    assert counts.tolist() == [k_sync, ei.value.required] and ei.value.required > 16
    assert int(small.tile_ranges.abs().sum()) == 0
    assert float(f.color.abs().max()) == 0.0 and bool((f.t_final == 1.0).all()) and int(f.n_trav.sum()) == 0
    assert float(g2.abs().max()) == 0.0


# ------------------------------------------------------------------ forward compositing

@pytest.mark.parametrize("name", ["tiny", "ragged_sh1", "ragged_sh2", "offscreen_sh3", "100k"])
@pytest.mark.parametrize("t_min", [1e-4, 0.0])
def test_forward_parity(name, t_min):
    log(f"forward parity {name} t_min={t_min}")
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree, t_min=t_min)
    st = gpu_forward(sc, cam, rp)
    op = oracle_params(rp)
    P = oracle.project(sc, cam, op)
    c, tf, nt, tie = oracle.render(P, op)
    ng = st.frame.n_trav.cpu().numpy()
    compare_images(st.frame.color.cpu().numpy(), st.frame.t_final.cpu().numpy(), c, tf, tie, ng, nt)
    log(f"  n_trav sum gpu={int(ng.sum())} orc={int(nt.sum())}")


# ------------------------------------------------------------------ loss

@pytest.mark.parametrize("h,w", [(64, 64), (37, 41), (1, 1), (1080, 1920)])
def test_loss_l1_parity(h, w):
    g = torch.Generator().manual_seed(h * 7 + w)
    c = torch.rand(h, w, 3, generator=g)
    t = torch.rand(h, w, 3, generator=g)
    t.view(-1)[::97] = c.view(-1)[::97]          # exact ties -> zero gradient
    loss_o, G_o = oracle.loss_l1(c, t)
    cg, tg = c.to(DEV), t.to(DEV)
    dl = torch.zeros_like(cg)
    loss = torch.zeros(1, device=DEV)
    ws = torch.empty(B.gs_loss_workspace_bytes(h * w), dtype=torch.uint8, device=DEV)
    B.gs_loss_l1(cg, tg, h * w, loss, dl, ws)
    torch.cuda.synchronize()
    assert abs(loss.item() - loss_o) <= 1e-6 * loss_o
    assert np.array_equal(dl.cpu().numpy().reshape(-1), G_o.astype(np.float32))


# ------------------------------------------------------------------ backward

def _ssim_pair(kind, h, w, seed):
    rng = np.random.default_rng(seed)
    x = rng.uniform(0.0, 1.0, size=(h, w, 3)).astype(np.float32)
    if kind == "random":
        y = rng.uniform(0.0, 1.0, size=(h, w, 3)).astype(np.float32)
    elif kind == "near":      # SSIM close to 1: small differences, small gradients
        y = np.clip(x + rng.normal(0.0, 0.01, size=x.shape), 0.0, 1.0).astype(np.float32)
    else:                     # smooth image with flat regions, against noise
        yy, xx = np.mgrid[0:h, 0:w]
        base = 0.5 + 0.4 * np.sin(xx / 13.0)[..., None] * np.cos(yy / 7.0)[..., None] * np.array([1.0, 0.6, 0.2])
        x = np.where(((xx // 20 + yy // 20) % 2 == 0)[..., None], base, 0.0).astype(np.float32)
        y = rng.uniform(0.0, 1.0, size=(h, w, 3)).astype(np.float32)
    return x, y


@pytest.mark.parametrize("h,w,lam,kind", [(64, 64, 0.2, "random"), (37, 41, 0.2, "near"), (1, 1, 0.2, "random"),
                                          (5, 130, 1.0, "smooth"), (16, 64, 0.0, "random"),
                                          (300, 257, 0.2, "smooth"), (1080, 1920, 0.2, "near")])
def test_loss_l1_dssim_parity(h, w, lam, kind):
    """(1 - lambda) L1 + lambda (1 - SSIM)/2 and dL/dC against the oracle's direct window sums
    (ROCm blog, "Why gsplat Cannot Just Use DDP"), over tiles, ragged edges and the
    one-pixel image.  Tolerances: the loss and SSIM within 2e-6; dL/dC within relative L2
    1e-4 of the oracle's, every element within 1e-3 of the largest; the L1 part's sign is
    decided in float32 on both sides."""
    log(f"L1 + D-SSIM {h}x{w} lambda={lam} {kind}")
    x, y = _ssim_pair(kind, h, w, h * 1000 + w)
    loss_o, G_o, ssim_o = oracle.loss_l1_dssim(x, y, lam)
    c, t = torch.from_numpy(x).to(DEV), torch.from_numpy(y).to(DEV)
    out = torch.full((2,), float("nan"), device=DEV)
    G = torch.full((h, w, 3), float("nan"), device=DEV)
    ws = torch.empty(B.gs_loss_l1_dssim_workspace_bytes(w, h), dtype=torch.uint8, device=DEV)
    B.gs_loss_l1_dssim(c, t, w, h, lam, out[0:1], out[1:2], G, ws)
    torch.cuda.synchronize()
    loss, ssim = float(out[0]), float(out[1])
    g = G.cpu().numpy().astype(np.float64)
    e = rel_l2(g, G_o)
    emax = float(np.abs(g - G_o).max() / max(np.abs(G_o).max(), 1e-30))
    log(f"  loss {loss:.8f} (oracle {loss_o:.8f}), SSIM {ssim:.8f} (oracle {ssim_o:.8f}), dL/dC rel-L2 {e:.2e}, "
        f"max {emax:.2e}")
    assert abs(loss - loss_o) <= 2e-6 and abs(ssim - ssim_o) <= 2e-6
    assert e <= 1e-4 and emax <= 1e-3
    # a second call gives the same bits (fixed summation order)
    G2 = torch.empty_like(G)
    out2 = torch.empty_like(out)
    B.gs_loss_l1_dssim(c, t, w, h, lam, out2[0:1], out2[1:2], G2, ws)
    torch.cuda.synchronize()
    assert torch.equal(G, G2) and torch.equal(out, out2)


def test_loss_l1_dssim_at_lambda_zero_is_the_l1_loss():
    """lambda = 0 reduces the objective to the L1 term: the gradient equals gs_loss_l1's bit
    for bit (sign(d) / (3 W H) either way)."""
    h, w = 45, 70
    x, y = _ssim_pair("random", h, w, 7)
    c, t = torch.from_numpy(x).to(DEV), torch.from_numpy(y).to(DEV)
    G0 = torch.empty(h, w, 3, device=DEV)
    G1 = torch.empty(h, w, 3, device=DEV)
    loss = torch.empty(2, device=DEV)
    ws = torch.empty(B.gs_loss_l1_dssim_workspace_bytes(w, h), dtype=torch.uint8, device=DEV)
    B.gs_loss_l1_dssim(c, t, w, h, 0.0, loss[0:1], None, G0, ws)
    lws = torch.empty(max(B.gs_loss_workspace_bytes(h * w), 8), dtype=torch.uint8, device=DEV)
    B.gs_loss_l1(c, t, h * w, loss[1:2], G1, lws)
    torch.cuda.synchronize()
    assert torch.equal(G0, G1)
    assert abs(float(loss[0]) - float(loss[1])) <= 1e-6 * float(loss[1])


@pytest.mark.parametrize("name", ["ragged_sh2", "100k"])
def test_dssim_training_step_gradients(name):
    """The training step with the structural term: forward, L1 + D-SSIM loss (lambda 0.2),
    backward rasterization, per-Gaussian sum and projection backward, against the oracle's
    render, orc_loss_l1_dssim gradient, raster backward and projection backward."""
    log(f"D-SSIM training step {name}")
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    op = oracle_params(rp)
    st = gpu_forward(sc, cam, rp)
    tgt = sc.targets[0]
    st.loss_dssim(tgt.to(DEV), 0.2)
    st.backward_partials(B.camera_from(cam))
    B.gs_grad_aggregate(st.params.gaussians(), st.proj.abi(), st.bins.abi(), B.camera_from(cam), rp, st.grads2d,
                        st.params.param_grads())
    torch.cuda.synchronize()
    P = oracle.project(sc, cam, op)
    c, tf, nt, tie = oracle.render(P, op)
    loss_o, G, ssim_o = oracle.loss_l1_dssim(c.astype(np.float32), tgt.numpy(), 0.2)
    assert abs(float(st.frame.loss) - loss_o) <= 1e-5 and abs(float(st.frame.ssim) - ssim_o) <= 1e-5
    g2_o = oracle.raster_backward(P, G, None, op)
    g3_o = oracle.project_backward(sc, cam, g2_o, op)
    g2 = st.grads2d.cpu().numpy()
    errs = {oracle.G_FIELDS[f]: rel_l2(g2[f], g2_o[f]) for f in range(9)}
    gp = st.params
    errs3 = {nm: rel_l2(gp.view(gp.grad, nm).cpu().numpy(), g3_o[nm]) for nm in
             ("means", "log_scales", "quats", "opacity_logits", "sh")}
    log(f"  loss {float(st.frame.loss):.6f} (oracle {loss_o:.6f}); grads2d rel-L2 max {max(errs.values()):.2e}; "
        f"grads3d rel-L2 max {max(errs3.values()):.2e}")
    assert max(errs.values()) <= 1e-3 and max(errs3.values()) <= 1e-3, (errs, errs3)


def _oracle_G(c_orc, target):
    """dL/dC of the L1 loss on the oracle's image, as the float32 input both sides use."""
    _, G = oracle.loss_l1(c_orc.astype(np.float32), target)
    return G.astype(np.float32).reshape(c_orc.shape)


@pytest.mark.parametrize("name", ["tiny", "ragged_sh1", "ragged_sh2", "offscreen_sh3", "100k"])
@pytest.mark.parametrize("with_gt", [False, True])
def test_backward_parity(name, with_gt):
    log(f"backward parity {name} with_gt={with_gt}")
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    op = oracle_params(rp)
    st = gpu_forward(sc, cam, rp)
    P = oracle.project(sc, cam, op)
    c, tf, nt, tie = oracle.render(P, op)
    G = _oracle_G(c, sc.targets[0].numpy())
    GT = None
    if with_gt:
        GT = (np.random.default_rng(5).normal(size=tf.shape) * 1e-4).astype(np.float32)
    g2_o = oracle.raster_backward(P, G.astype(np.float64), None if GT is None else GT.astype(np.float64), op)
    g3_o = oracle.project_backward(sc, cam, g2_o, op)
    Gd = torch.from_numpy(G).to(DEV)
    GTd = torch.from_numpy(GT).to(DEV) if GT is not None else None
    st.backward(B.camera_from(cam), dL_dcolor=Gd, dL_dt=GTd)
    torch.cuda.synchronize()
    g2 = st.grads2d.cpu().numpy()
    errs = {oracle.G_FIELDS[f]: rel_l2(g2[f], g2_o[f]) for f in range(9)}
    log(f"  grads2d rel-L2 {errs}")
    assert max(errs.values()) <= 1e-3, errs
    gp = st.params
    errs3 = {nm: rel_l2(gp.view(gp.grad, nm).cpu().numpy(), g3_o[nm]) for nm in
             ("means", "log_scales", "quats", "opacity_logits", "sh")}
    log(f"  grads3d rel-L2 {errs3}")
    assert max(errs3.values()) <= 1e-3, errs3
    # repeat: the per-Gaussian sums run in a fixed order, so the gradients are bit-identical;
    # grads2d and grads3d are written, not accumulated, so what they held before is irrelevant
    first = st.grads2d.clone()
    first3 = gp.grad.clone()
    st.grads2d.fill_(7.0)
    gp.grad.fill_(-3.0)
    st.backward(B.camera_from(cam), dL_dcolor=Gd, dL_dt=GTd)
    torch.cuda.synchronize()
    assert torch.equal(st.grads2d, first) and torch.equal(gp.grad, first3)


@pytest.mark.parametrize("with_gt", [False, True])
def test_backward_deep_stack_no_termination(with_gt):
    """theta_T = 0 over lists of ~1300 near-opaque entries: T_final is exactly 0 in float32
    at about 30% of the pixels (the oracle's, in double, is as small as 1e-231), so the
    front entries' T_i cannot be recovered from T_final; the backward must still match."""
    log(f"backward deep stack theta_T=0 with_gt={with_gt}")
    sc = scenes.scene_small_random(15, 3000, 72, 40, 1, extent=0.6, distance=3.0, log_scale_mean=-2.0,
                                   logit_mean=4.0)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree, t_min=0.0)
    op = oracle_params(rp)
    st = gpu_forward(sc, cam, rp)
    P = oracle.project(sc, cam, op)
    c, tf, nt, tie = oracle.render(P, op)
    assert (tf.astype(np.float32) == 0).mean() > 0.2     # the case this test is about
    compare_images(st.frame.color.cpu().numpy(), st.frame.t_final.cpu().numpy(), c, tf, tie,
                   st.frame.n_trav.cpu().numpy(), nt)
    G = _oracle_G(c, sc.targets[0].numpy())
    GT = (np.random.default_rng(6).normal(size=tf.shape)).astype(np.float32) if with_gt else None
    g2_o = oracle.raster_backward(P, G.astype(np.float64), None if GT is None else GT.astype(np.float64), op)
    st.backward(B.camera_from(cam), dL_dcolor=torch.from_numpy(G).to(DEV),
                dL_dt=torch.from_numpy(GT).to(DEV) if GT is not None else None, grads3d=False)
    torch.cuda.synchronize()
    g2 = st.grads2d.cpu().numpy()
    errs = {oracle.G_FIELDS[f]: rel_l2(g2[f], g2_o[f]) for f in range(9)}
    log(f"  grads2d rel-L2 {errs}")
    assert max(errs.values()) <= 1e-3, errs


def test_backward_split_matches_whole():
    """gs_raster_bwd_partials then gs_grad_aggregate gives gs_raster_bwd's gradients, bit for bit."""
    sc = SMALL["ragged_sh2"]()
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    st = gpu_forward(sc, cam, rp)
    c = B.camera_from(cam)
    G = torch.rand(cam.height, cam.width, 3, device=DEV) - 0.5
    GT = torch.rand(cam.height, cam.width, device=DEV) - 0.5
    st.backward(c, dL_dcolor=G, dL_dt=GT)
    whole2, whole3 = st.grads2d.clone(), st.params.grad.clone()
    st.grads2d.fill_(float("nan"))
    st.params.grad.fill_(float("nan"))
    f = st.frame
    g = st.params.gaussians()
    B.gs_raster_bwd_partials(g, st.bins.abi(), c, st.raster, f.color, f.t_final, f.n_trav, G, GT)
    B.gs_grad_aggregate(g, st.proj.abi(), st.bins.abi(), c, st.raster, st.grads2d, st.params.param_grads())
    torch.cuda.synchronize()
    assert torch.equal(st.grads2d, whole2) and torch.equal(st.params.grad, whole3)


@pytest.mark.parametrize("name", ["tiny", "ragged_sh1", "ragged_sh2", "offscreen_sh3", "100k"])
def test_fused_aggregate_adam_matches_separate_calls(name):
    """gs_grad_aggregate_adam equals gs_grad_aggregate -> gs_project_bwd -> gs_adam_step bit
    for bit (parameters, moments, screen-space gradients), over two steps."""
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    c = B.camera_from(cam)
    tgt = sc.targets[0].to(DEV)
    runs = []
    for fused in (False, True):
        st = gpu_forward(sc, cam, rp)
        for step in range(2):
            if step:
                st.forward(c)
            st.loss(tgt)
            if fused:
                st.backward_partials(c)
                st.aggregate_adam(c, grads2d=st.grads2d)
            else:
                st.backward(c)
                st.adam()
        torch.cuda.synchronize()
        runs.append((st.params.data.clone(), st.params.m.clone(), st.params.v.clone(), st.grads2d.clone()))
    (p0, m0, v0, g0), (p1, m1, v1, g1) = runs
    assert torch.equal(g0, g1)
    assert torch.equal(p0, p1) and torch.equal(m0, m1) and torch.equal(v0, v1)
    assert float((m1 != 0).float().mean()) > 0.0


def _moved_camera(cam):
    """The same camera shifted sideways and back (a second view of the scene)."""
    vm = cam.viewmat.clone().reshape(4, 4)
    vm[0, 3] += 0.15
    vm[2, 3] += 0.4
    return scenes._camera(vm.reshape(16).contiguous(), cam.width, cam.height)


def _proj_fields(pr):
    """depth, radii, the raster record, then the plain planes where the projection holds them."""
    return [t.clone() for t in (pr.depth, pr.radii, pr.rec, pr.means2d, pr.conic_opacity, pr.color)
            if t is not None]


@pytest.mark.parametrize("name", ["tiny", "ragged_sh1", "ragged_sh2", "offscreen_sh3", "100k"])
def test_fused_adam_projection_matches_separate_calls(name):
    """gs_grad_aggregate_adam_project equals gs_grad_aggregate_adam followed by gs_project of
    the updated Gaussians for the next camera, bit for bit (every projected field, the
    parameters and the Adam moments), over two steps on two views."""
    log(f"fused adam + next projection {name}")
    sc = _scene(name)
    cams = [sc.cameras[0], _moved_camera(sc.cameras[0])]
    rp = B.make_params(sc.sh_degree)
    tgt = sc.targets[0].to(DEV)
    runs = []
    for fused in (False, True):
        st = gpu_forward(sc, cams[0], rp)
        projs = []
        for step in range(2):
            c, nc = B.camera_from(cams[step % 2]), B.camera_from(cams[(step + 1) % 2])
            if step:
                st.forward_projected(c)
            st.loss(tgt)
            st.backward_partials(c)
            for t in (st.proj.means2d, st.proj.conic_opacity, st.proj.color, st.proj.depth, st.proj.rec):
                if t is not None:
                    t.fill_(-123.0)
            st.proj.radii.fill_(-5)
            if fused:
                st.aggregate_adam_project(c, nc)
            else:
                st.aggregate_adam(c)
                B.gs_project(st.params.gaussians(), nc, rp, st.proj.abi())
            torch.cuda.synchronize()
            projs.append(_proj_fields(st.proj))
        runs.append((projs, st.params.data.clone(), st.params.m.clone(), st.params.v.clone()))
    (pa, p0, m0, v0), (pb, p1, m1, v1) = runs
    for sa, sb in zip(pa, pb):
        for a, b in zip(sa, sb):
            assert torch.equal(a, b)
    assert torch.equal(p0, p1) and torch.equal(m0, m1) and torch.equal(v0, v1)
    # the projection saw the updated parameters: its visible records differ from view 0's
    assert int((pb[0][1][:, 0] > 0).sum()) > 0


def _owner_update_runs(sc, cams, rp, g2s, modes):
    """Two steps of the owner's update from the given screen-space gradients g2s[step] on the
    cameras cams[step % 2], each projecting for the other camera afterwards, per mode:
    "separate" (gs_project_bwd, gs_adam_step, gs_project), "fused_next" (gs_project_bwd_adam
    with next_cam) or "fused" (without; the projection then by gs_project).  Returns per mode
    the projections after each step, the parameters and moments, and m after the first step."""
    out = {}
    for mode in modes:
        params = PL.GaussianParams.from_scene(sc, DEV)
        st = PL.TrainStep(params, cams[0].width, cams[0].height, DEV, raster=rp, plain=True)
        projs, m_first = [], None
        for step in range(2):
            c, nc = B.camera_from(cams[step % 2]), B.camera_from(cams[(step + 1) % 2])
            g2 = g2s[step].to(DEV)
            for t in (st.proj.means2d, st.proj.conic_opacity, st.proj.color, st.proj.depth, st.proj.rec):
                t.fill_(-123.0)
            st.proj.radii.fill_(-5)
            if mode == "separate":
                B.gs_project_bwd(params.gaussians(), c, rp, g2, params.param_grads())
                st.adam()
            else:
                params.step_count += 1
                m, v = params.moments()
                nxt = mode == "fused_next"
                B.gs_project_bwd_adam(params.gaussians(), c, rp, g2, m, v, B.AdamLrs(**st.lr), params.step_count,
                                      0.9, 0.999, 1e-15, nc if nxt else None, st.proj.abi() if nxt else None)
            if mode != "fused_next":
                B.gs_project(params.gaussians(), nc, rp, st.proj.abi())
            torch.cuda.synchronize()
            assert torch.equal(g2.cpu(), g2s[step]), "the screen-space gradients are read, not modified"
            projs.append(_proj_fields(st.proj))
            if step == 0:
                m_first = params.m.clone()
        out[mode] = (projs, params.data.clone(), params.m.clone(), params.v.clone(), m_first, params)
    return out


@pytest.mark.parametrize("name", ["tiny", "ragged_sh1", "ragged_sh2", "offscreen_sh3", "100k"])
def test_owner_update_matches_separate_calls(name):
    """gs_project_bwd_adam (the owner's projection backward and Adam from decoded
    screen-space gradients, with or without the next camera's projection) equals
    gs_project_bwd, gs_adam_step and gs_project bit for bit: every projected field, the
    parameters and the moments, over two steps on two views.  Its 3D gradient, read back
    from m after the first step from zero moments (m = (1 - beta1) g), matches the oracle's
    projection backward of the same screen-space gradients."""
    log(f"owner update {name}")
    sc = _scene(name)
    cams = [sc.cameras[0], _moved_camera(sc.cameras[0])]
    rp = B.make_params(sc.sh_degree)
    gen = torch.Generator().manual_seed(len(name))
    g2s = [(torch.randn(9, sc.n, generator=gen) * 1e-3).contiguous() for _ in range(2)]
    runs = _owner_update_runs(sc, cams, rp, g2s, ("separate", "fused_next", "fused"))
    ref = runs["separate"]
    for mode in ("fused_next", "fused"):
        got = runs[mode]
        for sa, sb in zip(ref[0], got[0]):
            for a, b in zip(sa, sb):
                assert torch.equal(a, b), mode
        for a, b in zip(ref[1:5], got[1:5]):
            assert torch.equal(a, b), mode
    assert int((ref[0][0][1][:, 0] > 0).sum()) > 0
    g3 = oracle.project_backward(sc, cams[0], g2s[0].double().numpy(), oracle_params(rp))
    params = runs["fused_next"][5]
    g_dev = runs["fused_next"][4].cpu().numpy().astype(np.float64) / (1.0 - np.float32(0.9))
    for nm in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        e = rel_l2(params.view(torch.from_numpy(g_dev), nm).numpy(), g3[nm])
        log(f"  {name} {nm}: owner-update gradient vs oracle rel-L2 {e:.2e}")
        assert e <= 1e-3


def test_owner_update_large_blocks_match_separate_calls():
    """gs_project_bwd_adam above 2^22 Gaussians (the launch with 128-thread blocks): equal to
    gs_project_bwd, gs_adam_step and gs_project bit for bit; 2^22 + 4097 Gaussians, SH3."""
    n = (1 << 22) + 4097
    log(f"owner update, large blocks, n={n}")
    sc = scenes.scene_small_random(21, n, 320, 200, 3, extent=1.5, distance=3.0, log_scale_mean=-4.0)
    cams = [sc.cameras[0], _moved_camera(sc.cameras[0])]
    rp = B.make_params(sc.sh_degree)
    gen = torch.Generator().manual_seed(5)
    g2s = [(torch.randn(9, n, generator=gen) * 1e-3).contiguous() for _ in range(2)]
    runs = _owner_update_runs(sc, cams, rp, g2s, ("separate", "fused_next"))
    ref, got = runs["separate"], runs["fused_next"]
    for sa, sb in zip(ref[0], got[0]):
        for a, b in zip(sa, sb):
            assert torch.equal(a, b)
    for a, b in zip(ref[1:5], got[1:5]):
        assert torch.equal(a, b)


class _PlainParams(PL.GaussianParams):
    """The parameter store with plane stride n (no padding)."""
    LD_ALIGN = 1


@pytest.mark.parametrize("name", ["ragged_sh1", "ragged_sh2", "offscreen_sh3"])
def test_padded_plane_stride_equals_unpadded(name):
    """The padded parameter store (plane stride n rounded up to 64) and the plain one
    (stride n) give the same results bit for bit through every entry point that reads or
    writes parameter, gradient or moment planes: the one-view step with the fused end of step
    and the next projection, the projection backward into 3D gradients, the owner update
    and the batch step; ragged n, two steps."""
    log(f"padded vs plain plane stride {name}")
    sc = _scene(name)
    assert sc.n % 64 != 0
    cams = [sc.cameras[0], _moved_camera(sc.cameras[0])]
    bc = [B.camera_from(c) for c in cams]
    rp = B.make_params(sc.sh_degree)
    tgt = sc.targets[0].to(DEV)
    gen = torch.Generator().manual_seed(3)
    g2 = (torch.randn(9, sc.n, generator=gen) * 1e-3).contiguous().to(DEV)
    out = {}
    for cls in (PL.GaussianParams, _PlainParams):
        params = cls.from_scene(sc, DEV)
        assert params.ld == (sc.n if cls is _PlainParams else -(-sc.n // 64) * 64)
        st = PL.TrainStep(params, cams[0].width, cams[0].height, DEV, raster=rp, plain=True)
        st.forward(bc[0])
        res = []
        for step in range(2):
            if step:
                st.forward_projected(bc[step % 2])
            st.loss(tgt)
            st.backward_partials(bc[step % 2])
            st.aggregate_adam_project(bc[step % 2], bc[(step + 1) % 2])
            torch.cuda.synchronize()
            res += _proj_fields(st.proj)
        B.gs_project_bwd(params.gaussians(), bc[0], rp, g2, params.param_grads())
        params.step_count += 1
        m, v = params.moments()
        B.gs_project_bwd_adam(params.gaussians(), bc[1], rp, g2, m, v, B.AdamLrs(**st.lr), params.step_count, 0.9,
                              0.999, 1e-15, bc[0], st.proj.abi())
        torch.cuda.synchronize()
        res += [params.grad.clone()] + _proj_fields(st.proj)
        bt = PL.BatchTrainStep(params, cams[0].width, cams[0].height, 2, DEV, raster=rp)
        bt.project(bc)
        for k in range(2):
            bt.sort(k, bc[k])
            bt.render(k, bc[k], tgt)
        bt.update(bc, next_cams=bc)
        torch.cuda.synchronize()
        res += [params.data.clone(), params.m.clone(), params.v.clone()] + _proj_fields(bt.proj[1])
        pad = [params.store[k][:, params.n:] for k in ("data", "grad", "m", "v")]
        assert all(int((t != 0).sum()) == 0 for t in pad), "the padding stays zero"
        out[cls] = res
    a, b = out[PL.GaussianParams], out[_PlainParams]
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _views(cam, k):
    """k cameras: cam and copies moved sideways and back by growing amounts."""
    out = [cam]
    for j in range(1, k):
        vm = cam.viewmat.clone().reshape(4, 4)
        vm[0, 3] += 0.15 * j
        vm[1, 3] -= 0.05 * j
        vm[2, 3] += 0.3 * j
        out.append(scenes._camera(vm.reshape(16).contiguous(), cam.width, cam.height))
    return out


@pytest.mark.parametrize("name,views", [("tiny", 1), ("tiny", 4), ("ragged_sh1", 3), ("ragged_sh2", 2),
                                        ("offscreen_sh3", 4), ("100k", 4)])
def test_project_batch_matches_project(name, views):
    """gs_project_batch writes for every camera exactly what gs_project writes."""
    sc = _scene(name)
    cams = [B.camera_from(c) for c in _views(sc.cameras[0], views)]
    rp = B.make_params(sc.sh_degree)
    params = PL.GaussianParams.from_scene(sc, DEV)
    batch = [PL.Projection(sc.n, DEV, plain=(k % 2 == 0)) for k in range(len(cams))]
    B.gs_project_batch(params.gaussians(), cams, rp, [p.abi() for p in batch])
    for k, (c, pb) in enumerate(zip(cams, batch)):
        one = PL.Projection(sc.n, DEV, plain=(k % 2 == 0))
        B.gs_project(params.gaussians(), c, rp, one.abi())
        torch.cuda.synchronize()
        for a, b in zip(_proj_fields(one), _proj_fields(pb)):
            assert torch.equal(a, b)


def _batch_setup(sc, views, rp):
    """A BatchTrainStep with every view projected, binned and rendered (fused L1)."""
    cams = [B.camera_from(c) for c in _views(sc.cameras[0], views)]
    params = PL.GaussianParams.from_scene(sc, DEV)
    bt = PL.BatchTrainStep(params, sc.cameras[0].width, sc.cameras[0].height, views, DEV, raster=rp)
    bt.project(cams)
    tgt = sc.targets[0].to(DEV)
    for k, c in enumerate(cams):
        bt.sort(k, c)
        bt.render(k, c, tgt)
    torch.cuda.synchronize()
    return bt, cams


@pytest.mark.parametrize("name,views", [("tiny", 1), ("tiny", 4), ("ragged_sh1", 2), ("ragged_sh2", 4),
                                        ("offscreen_sh3", 2), ("100k", 4)])
def test_batch_end_of_step_matches_separate_calls(name, views):
    """gs_grad_aggregate_adam_batch equals, bit for bit, gs_grad_aggregate + gs_project_bwd per
    view, the 3D gradients scaled by 1/views and added in view order, gs_adam_step with the
    batch hyper-parameters, and gs_project_batch of the updated Gaussians for the next views
    (parameters, Adam moments and every projected field)."""
    log(f"batch end of step {name} views={views}")
    sc = _scene(name)
    rp = B.make_params(sc.sh_degree)
    bt, cams = _batch_setup(sc, views, rp)
    nxt = [B.camera_from(c) for c in _views(_moved_camera(sc.cameras[0]), views)]
    p0 = bt.params.data.clone()
    # separate calls on a copy of the parameters, reading the same slots
    ref = PL.GaussianParams.from_scene(sc, DEV)
    acc = torch.zeros_like(ref.grad)
    g2 = torch.zeros(9, max(sc.n, 1), device=DEV)
    for k, c in enumerate(cams):
        B.gs_grad_aggregate(ref.gaussians(), bt.proj[k].abi(), bt.bins[k].abi(), c, rp, g2, ref.param_grads())
        acc = acc + ref.grad * (1.0 / views)
    ref.grad.copy_(acc)
    lr_dict = {nm: getattr(bt.lrs, nm) for nm in PL.DEFAULT_LR}
    B.gs_adam_step(ref.adam_groups(lr_dict), 1, bt.beta1, bt.beta2, bt.eps)
    ref_proj = [PL.Projection(sc.n, DEV) for _ in nxt]
    B.gs_project_batch(ref.gaussians(), nxt, rp, [p.abi() for p in ref_proj])
    # the batched pass
    bt.update(cams, nxt)
    torch.cuda.synchronize()
    assert torch.equal(bt.params.data, ref.data)
    assert torch.equal(bt.params.m, ref.m) and torch.equal(bt.params.v, ref.v)
    assert not torch.equal(bt.params.data, p0)
    for a, b in zip(bt.proj, ref_proj):
        for x, y in zip(_proj_fields(a), _proj_fields(b)):
            assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["ragged_sh2", "100k"])
def test_batch_step_on_view_streams_matches_one_stream(name):
    """BatchTrainStep.step with each view binned and rasterized on its own stream gives, over
    three steps, the parameters, moments, images and losses of the same steps on one stream,
    bit for bit."""
    log(f"batch step on view streams {name}")
    sc = _scene(name)
    rp = B.make_params(sc.sh_degree)
    views = 4
    cams = [B.camera_from(c) for c in _views(sc.cameras[0], views)]
    tgt = sc.targets[0].to(DEV)
    out = []
    for concurrent in (False, True):
        bt, _ = _batch_setup(sc, views, rp)   # sized bins; projections for cams
        for b in bt.bins:
            b._alloc(int(b.capacity * 1.5) + 1024)
        vs = PL.ViewStreams(views) if concurrent else None
        for _ in range(3):
            bt.step(cams, [tgt] * views, next_cams=cams, view_streams=vs)
        torch.cuda.synchronize()
        out.append([bt.params.data.clone(), bt.params.m.clone(), bt.params.v.clone()]
                   + [f.color.clone() for f in bt.frame] + [f.loss.clone() for f in bt.frame])
    for a, b in zip(*out):
        assert torch.equal(a, b)


def test_batch_of_one_equals_single_view_pass():
    """A batch of one view with grad_scale 1 is gs_grad_aggregate_adam_project."""
    sc = _scene("ragged_sh2")
    rp = B.make_params(sc.sh_degree)
    bt, cams = _batch_setup(sc, 1, rp)
    nc = B.camera_from(_moved_camera(sc.cameras[0]))
    st = gpu_forward(sc, sc.cameras[0], rp)
    st.fused_l1(cams[0], sc.targets[0].to(DEV))
    st.aggregate_adam_project(cams[0], nc)
    bt.update(cams, [nc])
    torch.cuda.synchronize()
    assert torch.equal(bt.params.data, st.params.data) and torch.equal(bt.params.m, st.params.m)
    for x, y in zip(_proj_fields(bt.proj[0]), _proj_fields(st.proj)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["tiny", "ragged_sh2"])
def test_batch_gradient_matches_oracle(name):
    """The batch gradient is the mean of the views' gradients (each the oracle's backward of
    its own view): after one step from zero moments, m = (1 - beta1) g with the batch's
    beta1, so g is read back from m and compared with the oracle's mean."""
    views = 2
    sc = _scene(name)
    rp = B.make_params(sc.sh_degree)
    op = oracle_params(rp)
    cams = _views(sc.cameras[0], views)
    params = PL.GaussianParams.from_scene(sc, DEV)
    bt = PL.BatchTrainStep(params, cams[0].width, cams[0].height, views, DEV, raster=rp)
    bc = [B.camera_from(c) for c in cams]
    bt.project(bc)
    g3_sum = None
    for k, c in enumerate(cams):
        bt.sort(k, bc[k])
        P = oracle.project(sc, c, op)
        col, tf, nt, tie = oracle.render(P, op)
        G = _oracle_G(col, sc.targets[0].numpy())
        f = bt.frame[k]
        B.gs_raster_fwd(bt.proj[k].abi(), bt.bins[k].abi(), bc[k], rp, f.color, f.t_final, f.n_trav, f.n_trav_sum)
        B.gs_raster_bwd_partials(params.gaussians(), bt.bins[k].abi(), bc[k], rp, f.color, f.t_final, f.n_trav,
                                 torch.from_numpy(G).to(DEV), None)
        g3 = oracle.project_backward(sc, c, oracle.raster_backward(P, G.astype(np.float64), None, op), op)
        g3_sum = g3 if g3_sum is None else {nm: g3_sum[nm] + g3[nm] for nm in g3}
    bt.update(bc)
    torch.cuda.synchronize()
    g_batch = bt.params.m.cpu().numpy().astype(np.float64) / (1.0 - bt.beta1)
    for nm in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        got = params.view(torch.from_numpy(g_batch), nm).numpy()
        want = g3_sum[nm] / views
        e = rel_l2(got, want)
        log(f"  {name} {nm}: batch gradient vs oracle mean rel-L2 {e:.2e}")
        assert e <= 1e-3


# ------------------------------------------------------------------ Adam

@pytest.mark.parametrize("n,step", [(1, 1), (1001, 1), (4096, 7), (250_001, 3)])
def test_adam_parity(n, step):
    host = [(scenes.adam_state(n + step, n, step), 1e-3), (scenes.adam_state(n + step + 1, n + 3, step), 5e-2)]
    dev = [([t.to(DEV).contiguous() for t in st], lr) for st, lr in host]
    B.gs_adam_step([(p, g, m, v, lr) for (p, g, m, v), lr in dev], step, 0.9, 0.999, 1e-15)
    torch.cuda.synchronize()
    for ((p, g, m, v), lr), ((dp, dg, dm, dv), _) in zip(host, dev):
        assert torch.equal(dg.cpu(), g), "the gradients are read, not modified"
        po, mo, vo = oracle.adam(p, g, m, v, float(np.float32(lr)), float(np.float32(0.9)),
                                 float(np.float32(0.999)), float(np.float32(1e-15)), step)
        assert rel_l2(dp.cpu().numpy(), po) <= 1e-6
        assert rel_l2(dm.cpu().numpy(), mo) <= 1e-6
        assert rel_l2(dv.cpu().numpy(), vo) <= 1e-6
        # the update itself, not only the parameters
        upd_o = po - p.double().numpy()
        upd = dp.cpu().numpy().astype(np.float64) - p.double().numpy()
        assert rel_l2(upd, upd_o) <= 1e-4


@pytest.mark.parametrize("n", [1, 2, 5, 1001, 250_003])
def test_adam_groups_at_any_offset(n):
    """Parameter groups that are planes of [planes][n] buffers start at every offset from a
    16-byte boundary (n odd); each array's update still equals the oracle's.  The last
    group's gradient sits at another offset than its parameters (the scalar path)."""
    planes = 7
    st = scenes.adam_state(900 + n, planes * n, 4)
    bufs = [t.to(DEV).contiguous() for t in st]
    gshift = torch.zeros(planes * n + 1, device=DEV)
    gshift[1:] = bufs[1]
    bounds = [(0, 1), (1, 3), (3, 4), (4, 7)]
    groups = []
    for a, b in bounds[:-1]:
        groups.append((bufs[0][a * n:b * n], bufs[1][a * n:b * n], bufs[2][a * n:b * n], bufs[3][a * n:b * n], 1e-3))
    a, b = bounds[-1]
    groups.append((bufs[0][a * n:b * n], gshift[1 + a * n:1 + b * n], bufs[2][a * n:b * n], bufs[3][a * n:b * n], 1e-3))
    B.gs_adam_step(groups, 4, 0.9, 0.999, 1e-15)
    torch.cuda.synchronize()
    p, g, m, v = st
    po, mo, vo = oracle.adam(p, g, m, v, float(np.float32(1e-3)), float(np.float32(0.9)), float(np.float32(0.999)),
                             float(np.float32(1e-15)), 4)
    assert rel_l2(bufs[0].cpu().numpy(), po) <= 1e-6
    assert rel_l2(bufs[2].cpu().numpy(), mo) <= 1e-6
    assert rel_l2(bufs[3].cpu().numpy(), vo) <= 1e-6
    upd = bufs[0].cpu().numpy().astype(np.float64) - p.double().numpy()
    assert rel_l2(upd, po - p.double().numpy()) <= 1e-4
    # every element was updated exactly once: the moments match elementwise
    assert np.abs(bufs[2].cpu().numpy() - mo).max() <= 1e-6 * max(1.0, np.abs(mo).max())


# ------------------------------------------------------------------ partial renders

@pytest.mark.parametrize("parts,n_px,t_min", [(4, 5000, 1e-4), (4, 5000, 0.0), (1, 777, 1e-4), (3, 1, 1e-4)])
def test_composite_parity(parts, n_px, t_min):
    cs, ts = scenes.partial_images(20 + parts, parts, n_px)
    c_o, t_o = oracle.composite(cs, ts, float(np.float32(t_min)))
    cg = [c.to(DEV) for c in cs]
    tg = [t.to(DEV) for t in ts]
    c_out = torch.zeros(n_px, 3, device=DEV)
    t_out = torch.zeros(n_px, device=DEV)
    B.gs_composite_over(cg, tg, n_px, t_min, c_out, t_out)
    rng = np.random.default_rng(parts)
    G = rng.normal(size=(n_px, 3)).astype(np.float32)
    GT = rng.normal(size=n_px).astype(np.float32)
    dcs = [torch.zeros(n_px, 3, device=DEV) for _ in range(parts)]
    dts = [torch.zeros(n_px, device=DEV) for _ in range(parts)]
    B.gs_composite_over_bwd(cg, tg, n_px, t_min, torch.from_numpy(G).to(DEV), torch.from_numpy(GT).to(DEV), dcs, dts)
    torch.cuda.synchronize()
    assert np.abs(c_out.cpu().numpy() - c_o).max() <= 1e-6
    assert np.abs(t_out.cpu().numpy() - t_o).max() <= 1e-6
    dc_o, dt_o = oracle.composite_bwd(cs, ts, float(np.float32(t_min)), G, GT)
    for k in range(parts):
        assert np.abs(dcs[k].cpu().numpy() - dc_o[k]).max() <= 1e-5 * max(1, np.abs(dc_o[k]).max())
        assert np.abs(dts[k].cpu().numpy() - dt_o[k]).max() <= 1e-5 * max(1, np.abs(dt_o[k]).max())


@pytest.mark.parametrize("n,base", [(1, 0), (63, 5), (5000, 1000), (1_000_003, 7)])
def test_compact_bit_exact(n, base):
    g = scenes.sparse_grads(30 + n % 97, n)
    rec_o, bm_o = oracle.compact(g, base)
    gd = g.to(DEV)
    records = torch.zeros(n, 10, dtype=torch.int32, device=DEV)
    bitmap = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
    ws = torch.empty(B.gs_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    R = B.gs_compact_grads(gd, n, base, records, bitmap, ws)
    assert R == rec_o.shape[0]
    assert np.array_equal(records[:R].cpu().numpy().view(np.uint32), rec_o)
    assert np.array_equal(bitmap.cpu().numpy().view(np.uint32), bm_o)


def _shared_partitions(seed, n_owner, k, n_part_max, zero_frac=0.6):
    """k renderer partitions over an owner's n_owner Gaussians: each holds a random
    subset (positions in random order, so partitions overlap) with seeded sparse
    gradients; a few fields are subnormal."""
    rng = np.random.default_rng(seed)
    out = []
    for q in range(k):
        n_part = int(rng.integers(0, n_part_max + 1)) if q else n_part_max
        owner = rng.choice(n_owner, size=min(n_part, n_owner), replace=False).astype(np.uint32)
        g = scenes.sparse_grads(seed * 31 + q, len(owner), zero_frac=zero_frac)
        sub = torch.from_numpy(rng.random(g.shape) < 0.01) & (g != 0)
        g[sub] = torch.sign(g[sub]) * 1e-40
        out.append((g, owner, 1000 * q))
    return out


def _decode_both(parts, n_owner, init):
    """Compacts each partition on both sides (bit-identical, checked), then decodes on the
    GPU through the C ABI and in the oracle; returns (gpu [9][n_owner], oracle, count
    of contributions per owner Gaussian and field, sum of their magnitudes)."""
    gparts, oparts, keep = [], [], []
    for g, owner, base in parts:
        n = len(owner)
        rec_o, _ = oracle.compact(g, base)
        records = torch.zeros(max(n, 1), 10, dtype=torch.int32, device=DEV)
        bitmap = torch.zeros(max((n + 31) // 32, 1), dtype=torch.int32, device=DEV)
        ws = torch.empty(max(B.gs_compact_workspace_bytes(n), 256), dtype=torch.uint8, device=DEV)
        R = B.gs_compact_grads(g.to(DEV), n, base, records, bitmap, ws) if n else 0
        assert R == rec_o.shape[0]
        assert np.array_equal(records[:R].cpu().numpy().view(np.uint32), rec_o)
        om = torch.from_numpy(owner.astype(np.int64)).to(torch.int32).to(DEV) if n else None
        gparts.append((records, R, base, om, n))
        oparts.append((rec_o, base, owner, n))
        keep.append(records)
    out = init.clone().to(DEV)
    rejected = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.gs_decode_grads(gparts, out, n_owner, rejected)
    torch.cuda.synchronize()
    want, rej = oracle.decode(oparts, n_owner, out=init.numpy())
    assert rej == 0 and int(rejected.item()) == 0
    cnt = np.zeros((9, n_owner))
    mag = np.abs(init.numpy()).astype(np.float64)
    for rec_o, base, owner, n in oparts:
        pos = rec_o[:, 0].astype(np.int64) - base
        vals = rec_o[:, 1:].view(np.float32).T.astype(np.float64)
        np.add.at(cnt, (slice(None), owner[pos]), (vals != 0).astype(np.float64))
        np.add.at(mag, (slice(None), owner[pos]), np.abs(vals))
    return out.cpu().numpy(), want, cnt, mag


@pytest.mark.parametrize("seed,n_owner,k,n_part_max", [(1, 1, 1, 1), (2, 5000, 3, 4000), (3, 100_003, 5, 60_000),
                                                        (4, 2000, 16, 2000), (5, 300_000, 2, 300_000)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_decode_matches_oracle(seed, n_owner, k, n_part_max, accumulate):
    """ByteSplat section 6.2: the owner's gradients are the sum of every partition's
    records mapped through its forward index.  Bound: an fp32 sum of m terms onto the
    initial value errs by at most m u sum|terms| (u = 2^-24), plus 2^-126 per add if the
    atomic flushes subnormals; a Gaussian with a single normal-valued contribution onto
    zero is exact."""
    parts = _shared_partitions(seed, n_owner, k, n_part_max)
    init = torch.zeros(9, n_owner)
    if accumulate:
        init = torch.from_numpy(np.random.default_rng(seed).normal(size=(9, n_owner)).astype(np.float32))
    got, want, cnt, mag = _decode_both(parts, n_owner, init)
    m = cnt + (init.numpy() != 0)
    bound = m * (2.0 ** -24 * mag + 2.0 ** -126)
    err = np.abs(got.astype(np.float64) - want)
    assert (err <= bound).all(), float((err - bound).max())
    single = (cnt == 1) & (init.numpy() == 0) & (np.abs(want) >= 2.0 ** -126)
    assert np.array_equal(got[single], want[single].astype(np.float32))
    log(f"  decode k={k} owner={n_owner}: {int(cnt.sum())} adds, max sharing {int(cnt.max(initial=0))}")


def test_decode_rejected_and_empty():
    """Records outside their partition, or mapped outside the owner range, are skipped
    and counted; empty partitions and k = 0 do nothing."""
    n = 3000
    g = scenes.sparse_grads(7, n, zero_frac=0.0)
    records = torch.zeros(n, 10, dtype=torch.int32, device=DEV)
    bitmap = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
    ws = torch.empty(B.gs_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    R = B.gs_compact_grads(g.to(DEV), n, 500, records, bitmap, ws)
    assert R == n
    owner = np.arange(2000, dtype=np.uint32)
    owner[:7] = 4000                                   # past the owner range
    om = torch.from_numpy(owner.astype(np.int64)).to(torch.int32).to(DEV)
    out = torch.zeros(9, 2500, device=DEV)
    rejected = torch.zeros(1, dtype=torch.int32, device=DEV)
    empty = torch.zeros(1, 10, dtype=torch.int32, device=DEV)
    B.gs_decode_grads([(records, R, 500, om, 2000), (empty, 0, 0, None, 0)], out, 2500, rejected)
    B.gs_decode_grads([], out, 2500, rejected)
    torch.cuda.synchronize()
    assert int(rejected.item()) == 1000 + 7
    rec_o, _ = oracle.compact(g, 500)
    want, rej = oracle.decode([(rec_o, 500, owner, 2000)], 2500)
    assert rej == 1007
    assert np.array_equal(out.cpu().numpy(), want.astype(np.float32))


# ------------------------------------------------------------------ whole step, edge cases

def test_empty_scene_and_train_step():
    sc = scenes.scene_small_random(40, 0, 40, 24, 0)
    cam = sc.cameras[0]
    params = PL.GaussianParams.from_scene(sc, DEV)
    st = PL.TrainStep(params, cam.width, cam.height, DEV)
    st.step(B.camera_from(cam), sc.targets[0].to(DEV))
    torch.cuda.synchronize()
    assert st.bins.n_isect == 0
    assert float(st.frame.t_final.min()) == 1.0 and float(st.frame.color.abs().max()) == 0.0


def test_train_step_composition():
    """step() is exactly forward + loss + backward + adam (same kernels, same order)."""
    sc = scenes.scene_small_random(41, 800, 80, 64, 2, extent=1.0)
    cam = B.camera_from(sc.cameras[0])
    tgt = sc.targets[0].to(DEV)
    a = PL.TrainStep(PL.GaussianParams.from_scene(sc, DEV), 80, 64, DEV)
    b = PL.TrainStep(PL.GaussianParams.from_scene(sc, DEV), 80, 64, DEV)
    for _ in range(3):
        a.step(cam, tgt)
        b.forward(cam)
        b.loss(tgt)
        b.backward(cam)
        b.adam()
    torch.cuda.synchronize()
    assert rel_l2(a.params.data.cpu().numpy(), b.params.data.cpu().numpy()) <= 1e-6
    assert a.frame.loss.item() > 0


@pytest.mark.parametrize("name", ["ragged_sh1", "100k"])
def test_ntrav_sum(name):
    """The optional device sum of N_p equals the sum of the per-pixel counts, for a
    16-byte aligned n_trav and for one that is not (an odd pixel count leaves a tail)."""
    log(f"n_trav sum {name}")
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    st = gpu_forward(sc, cam, rp)
    c = B.camera_from(cam)
    f = st.frame
    want = int(f.n_trav.to(torch.int64).sum())
    assert want > 0
    tot = torch.zeros(1, dtype=torch.int64, device=DEV)
    B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), c, rp, f.color, f.t_final, f.n_trav, tot)
    buf = torch.full((cam.height * cam.width + 1,), -1, dtype=torch.int32, device=DEV)
    shifted = buf[1:].view(cam.height, cam.width)   # 4 bytes past a 256-byte boundary
    tot2 = torch.full((1,), 5, dtype=torch.int64, device=DEV)
    B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), c, rp, f.color, f.t_final, shifted, tot2)
    torch.cuda.synchronize()
    assert torch.equal(shifted, f.n_trav)
    assert int(tot) == want and int(tot2) == want + 5


# ------------------------------------------------------------------ fused forward + L1 + backward

@pytest.mark.parametrize("name,t_min", [("tiny", 1e-4), ("tiny", 0.0), ("ragged_sh1", 1e-4), ("ragged_sh2", 1e-4),
                                        ("offscreen_sh3", 1e-4), ("100k", 1e-4)])
def test_fused_l1_matches_separate_calls(name, t_min):
    """gs_raster_fused_l1 equals gs_raster_fwd -> gs_loss_l1 -> gs_raster_bwd_partials bit for
    bit: image, T_final, N_p, and the per-Gaussian sums of the gradient slots; the loss up
    to the order of its double sum; the same sum of N_p."""
    log(f"fused fwd + L1 + bwd {name} t_min={t_min}")
    sc = _scene(name)
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree, t_min=t_min)
    c = B.camera_from(cam)
    tgt = sc.targets[0].to(DEV)
    st = gpu_forward(sc, cam, rp)
    f = st.frame
    g = st.params.gaussians()
    f.n_trav_sum.zero_()
    B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), c, rp, f.color, f.t_final, f.n_trav, f.n_trav_sum)
    st.loss(tgt)
    st.backward_partials(c)
    B.gs_grad_aggregate(g, st.proj.abi(), st.bins.abi(), c, rp, st.grads2d, None)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (f.color, f.t_final, f.n_trav, st.grads2d, f.loss, f.n_trav_sum)]
    f.color.fill_(float("nan")); f.t_final.fill_(float("nan")); f.n_trav.fill_(-1)
    f.loss.fill_(float("nan")); f.n_trav_sum.zero_(); st.grads2d.fill_(float("nan"))
    st.fused_l1(c, tgt)
    B.gs_grad_aggregate(g, st.proj.abi(), st.bins.abi(), c, rp, st.grads2d, None)
    torch.cuda.synchronize()
    for a, b in zip((f.color, f.t_final, f.n_trav, st.grads2d), ref[:4]):
        assert torch.equal(a, b)
    assert int(f.n_trav_sum) == int(ref[5]) > 0
    assert abs(float(f.loss) - float(ref[4])) <= 1e-6 * abs(float(ref[4]))
    assert float(st.grads2d.abs().max()) > 0.0


def test_fused_l1_then_fused_adam_projection_matches_separate_step():
    """A whole fused step (bin sort, fused forward + L1 + backward, fused end of step with the
    next view's projection) equals the separate calls over two steps, bit for bit."""
    sc = _scene("ragged_sh2")
    cams = [sc.cameras[0], _moved_camera(sc.cameras[0])]
    rp = B.make_params(sc.sh_degree)
    tgt = sc.targets[0].to(DEV)
    out = []
    for fused in (False, True):
        st = gpu_forward(sc, cams[0], rp)
        for step in range(2):
            c, nc = B.camera_from(cams[step % 2]), B.camera_from(cams[(step + 1) % 2])
            if fused:
                if step:
                    st.bins.sort(st.proj, c, rp)
                st.fused_l1(c, tgt)
                st.aggregate_adam_project(c, nc)
            else:
                if step:
                    st.forward(c)
                st.loss(tgt)
                st.backward_partials(c)
                st.aggregate_adam(c)
        torch.cuda.synchronize()
        out.append((st.frame.color.clone(), st.params.data.clone(), st.params.m.clone(), st.params.v.clone()))
    for a, b in zip(*out):
        assert torch.equal(a, b)


def test_bin_sort_graph_replays_match_eager():
    """The binning captured as one HIP graph per view and replayed, with eager
    rasterization and host synchronisations between the replays, gives the eager sort's
    lists, counts and rendered images bit for bit on every replay."""
    log("bin sort graph replays")
    sc = _scene("ragged_sh2")
    cams = [B.camera_from(c) for c in (sc.cameras[0], _moved_camera(sc.cameras[0]))]
    rp = B.make_params(sc.sh_degree)
    tgt = sc.targets[0].to(DEV)
    st = gpu_forward(sc, sc.cameras[0], rp)
    st.bins._alloc(int(st.bins.capacity * 1.5) + 1024)
    projs = [st.proj, PL.Projection(sc.n, DEV)]
    B.gs_project(st.params.gaussians(), cams[1], rp, projs[1].abi())
    f = st.frame

    def outputs(v):
        k = int(st.bins.raster[:16].view(torch.int64)[0])
        return [st.bins.ids[:k].clone(), st.bins.tile_ranges.clone(), f.color.clone(), f.t_final.clone(),
                f.n_trav.clone(), f.loss.clone()]

    want, ks = [], []
    for v in range(2):
        n = torch.zeros(2, dtype=torch.int64, device=DEV)
        st.bins.sort_async(projs[v], cams[v], rp, n)
        st.fused_l1(cams[v], tgt)
        torch.cuda.synchronize()
        assert int(n[1]) == 0 and int(n[0]) > 0
        ks.append(int(n[0]))
        want.append(outputs(v))
    assert not torch.equal(want[0][2], want[1][2])
    counts = torch.full((2, 2), -1, dtype=torch.int64, device=DEV)
    acc = torch.zeros(2, dtype=torch.int64, device=DEV)
    graphs = [PL.BinSortGraph(st.bins, projs[v], cams[v], rp, counts[v], acc) for v in range(2)]
    acc.zero_()
    replays = 0
    for rnd in range(3):
        for v in (1, 0) if rnd % 2 else (0, 1):
            counts[v].fill_(-1)
            graphs[v].replay()
            st.fused_l1(cams[v], tgt)
            torch.cuda.synchronize()
            replays += 1
            assert counts[v].tolist() == [ks[v], 0]
            for a, b in zip(outputs(v), want[v]):
                assert torch.equal(a, b), f"replay {replays} of view {v} differs from the eager sort"
    assert acc.tolist() == [3 * (ks[0] + ks[1]), 0]
    # the graphs hold the buffers' addresses: after the binning buffers are replaced, a replay
    # is refused instead of writing into freed memory
    st.bins._alloc(st.bins.capacity + 4096)
    with pytest.raises(RuntimeError, match="reallocated"):
        graphs[0].replay()


def test_tile_budget_report():
    """ByteSplat Eq. 8 and Eq. 9 per tile against numpy on the tile lists of a sorted scene."""
    sc = _scene("100k")
    cam = sc.cameras[0]
    rp = B.make_params(sc.sh_degree)
    st = gpu_forward(sc, cam, rp)
    T = st.bins.tiles
    rng = st.bins.tile_ranges.cpu().numpy().astype(np.int64)
    nt = rng[1:] - rng[:-1]
    budget = int(np.percentile(nt[nt > 0], 60))
    excess = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    frac = torch.full((T,), -1.0, dtype=torch.float32, device=DEV)
    totals = torch.zeros(2, dtype=torch.int64, device=DEV)
    B.gs_tile_budget_report(st.bins.abi(), B.camera_from(cam), budget, excess, frac, totals)
    torch.cuda.synchronize()
    e = np.maximum(0, nt - budget)
    p = np.where(nt > 0, e / np.maximum(nt, 1), 0.0).astype(np.float32)
    assert np.array_equal(excess.cpu().numpy(), e.astype(np.int32))
    assert np.array_equal(frac.cpu().numpy(), p)
    assert totals.tolist() == [int((e > 0).sum()), int(e.sum())] and int((e > 0).sum()) > 0


# ------------------------------------------------------------------ reused raster buffers

_EPOCH_BYTE = 20   # BinsHeader: K (8 B), Q (8 B), ok (4 B), epoch (4 B)


@pytest.mark.parametrize("fused", [False, True])
def test_reused_raster_buffer_gives_fresh_gradients(fused):
    """The raster buffer may hold anything before a sort: here the stamps of three
    backward calls on another view's lists (epochs 2, 3, 4, on slots the second view's
    records also use), and a header epoch reset as if the memory had been reused, so that
    the second view's backward stamps with an epoch the stale slots already carry.  The
    second view's screen-space gradients must equal, bit for bit, those of a run on a
    zero-filled buffer, on the separate path (forward, L1, backward partials) and the
    fused one."""
    log(f"reused raster buffer, fused={fused}")
    sc = _scene("100k")
    cams = [sc.cameras[0], _moved_camera(sc.cameras[0])]
    rp = B.make_params(sc.sh_degree)
    c = [B.camera_from(x) for x in cams]
    tgt = sc.targets[0].to(DEV)
    W, H = cams[0].width, cams[0].height
    params = PL.GaussianParams.from_scene(sc, DEV)
    projs = [PL.Projection(sc.n, DEV) for _ in cams]
    for p, cc in zip(projs, c):
        B.gs_project(params.gaussians(), cc, rp, p.abi())
    # capacity for both views
    probe = PL.Binning(sc.n, W, H, device=DEV)
    probe.sort(projs[0], c[0], rp)
    probe.sort(projs[1], c[1], rp)
    cap = probe.capacity   # grown until both views' lists fit
    del probe

    def run(bins, view, poison):
        st = PL.TrainStep(params, W, H, DEV, raster=rp)
        st.bins, st.proj = bins, projs[view]
        if poison:
            # view 0's lists, three backward calls (the slots they write are stamped 2, 3, 4)
            bins.sort(projs[0], c[0], rp)
            B.gs_raster_fwd(projs[0].abi(), bins.abi(), c[0], rp, st.frame.color, st.frame.t_final,
                            st.frame.n_trav, None)
            st.loss(tgt)
            for _ in range(3):
                st.backward_partials(c[0])
        bins.sort(projs[view], c[view], rp)
        hdr = bins.raster[:32].view(torch.int32)
        assert int(hdr[_EPOCH_BYTE // 4]) == 1, "the sort starts the slot epochs at 1"
        hdr[_EPOCH_BYTE // 4] = 1   # a header reset as if the memory had been reused
        if fused:
            st.fused_l1(c[view], tgt)
        else:
            B.gs_raster_fwd(projs[view].abi(), bins.abi(), c[view], rp, st.frame.color, st.frame.t_final,
                            st.frame.n_trav, None)
            st.loss(tgt)
            st.backward_partials(c[view])
        B.gs_grad_aggregate(params.gaussians(), projs[view].abi(), bins.abi(), c[view], rp, st.grads2d, None)
        torch.cuda.synchronize()
        return st.grads2d.clone(), st.frame.color.clone()

    reused = PL.Binning(sc.n, W, H, capacity=cap, device=DEV)
    g_reused, img_reused = run(reused, 1, poison=True)
    fresh = PL.Binning(sc.n, W, H, capacity=cap, device=DEV)
    fresh.raster.zero_()
    g_fresh, img_fresh = run(fresh, 1, poison=False)
    assert torch.equal(img_reused, img_fresh)
    assert float(g_fresh.abs().max()) > 0.0
    diff = int((g_reused != g_fresh).sum())
    assert diff == 0, f"{diff} gradient values differ from the run on a zero-filled buffer"
