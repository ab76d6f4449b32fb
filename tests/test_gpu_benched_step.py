"""Oracle parity of the training step as bench.py times it.  GPU only.

The step is: the binning replayed as a per-view HIP graph (gs_bin_sort_async) ->
gs_raster_fused_l1 (forward, L1 loss and per-record backward in one kernel) ->
gs_grad_aggregate_adam_project (per-Gaussian sum, projection backward, Adam and the next
view's projection in one pass), over the 1M-Gaussian SH3 1080p scene's four views in
turn, from zero Adam moments.  Between the fused raster call and the end-of-step pass a
gs_grad_aggregate call (it only reads the gradient slots) captures the screen-space
gradients; nothing else is added to the step.

Per step, against the oracle run on the parameters the GPU held before the step:
* the projected records the step started from (gs_project for the first step, the
  previous step's fused projection after that);
* the whole 1920x1080 image, T_final and N_p;
* the screen-space gradients (ByteSplat Eq. 3-4) with the oracle's own L1 gradient;
* the 3D gradients, read back from the Adam moments: g = (m_t - beta1 m_{t-1}) / (1 - beta1);
* the Adam update of every parameter group from those gradients.

At 10M (skewed, 4K) the same fused calls run once on one view, which takes the end-of-step
kernel's wide-block variant (more than 2^22 Gaussians); the L1 target equals the GPU's own
render outside two bands of rows, so dL/dC = sign(0) = 0 there and the oracle can compare
the gradients of the band pixels.
"""
import concurrent.futures as cf
import gc

import numpy as np
import pytest
import torch

import oracle
from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import pipeline as PL
from differentiable_rasterization_amd import scenes
from tests.gpu_util import DEV, compare_images, compare_projection, log, oracle_params, rel_l2

pytestmark = pytest.mark.gpu

GROUPS = (("means", 0, 3), ("log_scales", 3, 6), ("quats", 6, 10), ("opacity_logits", 10, 11),
          ("sh_dc", 11, 14), ("sh_rest", 14, None))
# the hyper-parameters as the ABI receives them (float32): the oracle's Adam gets the same
# inputs, so (1 - beta2) is the float difference 1 - fl(0.999), as on the GPU
BETA1, BETA2, EPS = (float(np.float32(x)) for x in (0.9, 0.999, 1e-15))


def _scene_with(sc, planes):
    """The scene with the parameters of a GaussianParams buffer (CPU float32 [planes][N])."""
    p = planes.contiguous()
    return scenes.Scene(sc.name, sc.sh_degree, p[0:3].contiguous(), p[3:6].contiguous(), p[6:10].contiguous(),
                        p[10].contiguous(), p[11:].contiguous(), sc.cameras, sc.targets)


def _oracle_view(sc, planes, cam, target, op, pixels=None):
    """Projection, render, L1 gradient (of the oracle's image), screen-space and 3D
    gradients of one view; pixels restricts render and backward to those pixels."""
    s = _scene_with(sc, planes)
    P = oracle.project(s, cam, op)
    col, tf, nt, tie = oracle.render(P, op, pixels=pixels)
    tg = target if pixels is None else target[pixels[:, 1], pixels[:, 0]]
    _, G = oracle.loss_l1(col.astype(np.float32), tg)
    if pixels is not None:
        # the gradient of the band pixels' L1 term as the GPU's full-image mean sees it
        G = G * (len(pixels) / float(cam.width * cam.height))
    g2 = oracle.raster_backward(P, G.reshape(-1, 3), None, op, pixels=pixels)
    g3 = oracle.project_backward(s, cam, g2, op)
    return dict(P=P, color=col, t_final=tf, n_trav=nt, tie=tie, grads2d=g2, grads3d=g3)


def _check_grads2d(g2_gpu, g2_orc, what):
    errs = {oracle.G_FIELDS[f]: rel_l2(g2_gpu[f], g2_orc[f]) for f in range(9)}
    log(f"  {what} grads2d rel-L2 max {max(errs.values()):.2e} {errs}")
    assert max(errs.values()) <= 1e-3, errs


def _check_grads3d_and_adam(p0, m0, v0, p1, m1, v1, g3o, step, lrs, what, idx=None):
    """3D gradients from the moments against the oracle's; the Adam update of each group
    (oracle.adam from the same p, m, v and those gradients) against the GPU's."""
    g_gpu = (m1.astype(np.float64) - BETA1 * m0.astype(np.float64)) / (1.0 - BETA1)
    full = {nm: g3o[nm] for nm in ("means", "log_scales", "quats", "opacity_logits", "sh")}
    orc_planes = np.concatenate([full["means"], full["log_scales"], full["quats"],
                                 full["opacity_logits"][None], full["sh"]], axis=0)
    if idx is not None:
        orc_planes = orc_planes[:, idx]
    e3 = {}
    for nm, a, b in GROUPS:
        e3[nm] = rel_l2(g_gpu[a:b], orc_planes[a:b])
    log(f"  {what} grads3d (from m) rel-L2 max {max(e3.values()):.2e} {e3}")
    assert max(e3.values()) <= 1e-3, e3
    worst = 0.0
    for nm, a, b in GROUPS:
        po, mo, vo = oracle.adam(p0[a:b], g_gpu[a:b], m0[a:b], v0[a:b], float(np.float32(lrs[nm])), BETA1, BETA2,
                                 EPS, step)
        shape = p0[a:b].shape
        for got, want, lab in ((p1[a:b], po, "p"), (m1[a:b], mo, "m"), (v1[a:b], vo, "v")):
            e = rel_l2(got, want.reshape(shape))
            worst = max(worst, e)
            assert e <= 1e-6, (nm, lab, e)
        # the update itself, element by element: within 2 float32 ulps of the parameter plus
        # 1e-5 of the step (the gradient read back from m carries m's rounding into v)
        po = po.reshape(shape)
        ulp = np.spacing(np.abs(po).astype(np.float32)).astype(np.float64)
        slack = 2 * ulp + 1e-5 * np.abs(po - p0[a:b].astype(np.float64)) + 1e-30
        assert (np.abs(p1[a:b].astype(np.float64) - po) <= slack).all(), nm
    log(f"  {what} Adam p, m, v rel max {worst:.2e}")


def test_1m_1080p_benched_step_against_oracle():
    log("1M 1080p: the benched step (graph binning -> fused raster + L1 -> fused end of step) x 4 views")
    sc = scenes.scene_1m_1080p()
    cams = [B.camera_from(c) for c in sc.cameras]
    targets = [t.to(DEV) for t in sc.targets]
    nviews = len(cams)
    W, H = sc.cameras[0].width, sc.cameras[0].height
    params = PL.GaussianParams.from_scene(sc, DEV)
    st = PL.TrainStep(params, W, H, DEV)
    rp = st.raster
    op = oracle_params(rp)
    # as bench.py: size the lists for every view, grow them, capture each view's binning
    for c in cams:
        st.forward(c)
    st.bins._alloc(int(st.bins.capacity * 1.3) + 4096)
    torch.cuda.synchronize()
    view_counts = torch.zeros(nviews, 2, dtype=torch.int64, device=DEV)
    acc = torch.zeros(2, dtype=torch.int64, device=DEV)
    B.gs_project(params.gaussians(), cams[0], rp, st.proj.abi())
    graphs = [PL.BinSortGraph(st.bins, st.proj, cams[v], rp, view_counts[v], acc) for v in range(nviews)]
    B.gs_project(params.gaussians(), cams[0], rp, st.proj.abi())   # the first step's records
    g2_cap = torch.zeros(9, sc.n, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    cpu = lambda t: t.detach().cpu().numpy().copy()
    steps = []
    for i in range(nviews):
        c, t, nc = cams[i], targets[i], cams[(i + 1) % nviews]
        before = dict(p=cpu(params.data), m=cpu(params.m), v=cpu(params.v),
                      proj=PL.Projection(sc.n, DEV))
        for a, b in zip((before["proj"].depth, before["proj"].radii, before["proj"].rec),
                        (st.proj.depth, st.proj.radii, st.proj.rec)):
            a.copy_(b)
        graphs[i].replay()
        st.fused_l1(c, t)
        B.gs_grad_aggregate(params.gaussians(), st.proj.abi(), st.bins.abi(), c, rp, g2_cap, None)
        st.aggregate_adam_project(c, nc)
        torch.cuda.synchronize()
        assert view_counts[i].tolist()[1] == 0, "the lists must fit"
        steps.append(dict(before=before, color=cpu(st.frame.color), t_final=cpu(st.frame.t_final),
                          n_trav=cpu(st.frame.n_trav), g2=cpu(g2_cap), p1=cpu(params.data), m1=cpu(params.m),
                          v1=cpu(params.v), step=params.step_count))
        log(f"  GPU step {i}: K = {int(view_counts[i, 0])}, loss {float(st.frame.loss):.6f}")
    # the oracle of the four views in parallel (ctypes releases the GIL in the C oracle)
    with cf.ThreadPoolExecutor(max_workers=nviews) as ex:
        futs = [ex.submit(_oracle_view, sc, torch.from_numpy(steps[i]["before"]["p"]), sc.cameras[i],
                          sc.targets[i].numpy(), op) for i in range(nviews)]
        orcs = [f.result() for f in futs]
    log("  oracle done")
    lrs = dict(PL.DEFAULT_LR)
    for i, (s, o) in enumerate(zip(steps, orcs)):
        what = f"step {i} (view {i})"
        ps = compare_projection(s["before"]["proj"], o["P"])
        log(f"  {what} records the step started from: {ps}")
        compare_images(s["color"], s["t_final"], o["color"], o["t_final"], o["tie"], s["n_trav"], o["n_trav"],
                       label=f"1M 1080p benched step {i}")
        _check_grads2d(s["g2"], o["grads2d"], what)
        _check_grads3d_and_adam(s["before"]["p"], s["before"]["m"], s["before"]["v"], s["p1"], s["m1"],
                                s["v1"], o["grads3d"], s["step"], lrs, what)
    # the last step's fused projection (for view 0 of the next round) against the oracle
    P = oracle.project(_scene_with(sc, torch.from_numpy(steps[-1]["p1"])), sc.cameras[0], op)
    log(f"  next view's records after the last step: {compare_projection(st.proj, P)}")
    del st, params, graphs
    gc.collect()
    torch.cuda.empty_cache()


def _band(width, y0, rows):
    return np.stack([np.tile(np.arange(width, dtype=np.int32), rows),
                     np.repeat(np.arange(y0, y0 + rows, dtype=np.int32), width)], axis=1).copy()


def test_10m_4k_fused_step_bands_against_oracle():
    log("10M 4K skewed: fused raster + L1 -> fused end of step (wide-block variant), bands vs oracle")
    sc = scenes.scene_skewed_4k()
    cam = sc.cameras[0]
    c = B.camera_from(cam)
    W, H = cam.width, cam.height
    params = PL.GaussianParams.from_scene(sc, DEV)
    st = PL.TrainStep(params, W, H, DEV)
    rp = st.raster
    op = oracle_params(rp)
    st.forward(c)
    torch.cuda.synchronize()
    bands = [(1072, 6), (300, 3)]
    pix = np.concatenate([_band(W, y0, rows) for y0, rows in bands])
    # L1 target: the GPU's own render (dL/dC = 0) except on the band rows
    tgt = st.frame.color.clone()
    for y0, rows in bands:
        tgt[y0:y0 + rows] = sc.targets[0][y0:y0 + rows].to(DEV)
    ref_color = st.frame.color.clone()
    p0, m0, v0 = (x.cpu().numpy().copy() for x in (params.data, params.m, params.v))
    g2_cap = torch.zeros(9, sc.n, dtype=torch.float32, device=DEV)
    st.fused_l1(c, tgt)
    B.gs_grad_aggregate(params.gaussians(), st.proj.abi(), st.bins.abi(), c, rp, g2_cap, None)
    st.aggregate_adam_project(c, c)
    torch.cuda.synchronize()
    assert torch.equal(st.frame.color, ref_color), "the fused forward must equal the separate one"
    color = st.frame.color.cpu().numpy()
    tf = st.frame.t_final.cpu().numpy()
    nt = st.frame.n_trav.cpu().numpy()
    g2 = g2_cap.cpu().numpy()
    p1, m1, v1 = (x.cpu().numpy() for x in (params.data, params.m, params.v))
    log("  oracle: projection, band render and backward, projection backward")
    P = oracle.project(sc, cam, op)
    col_o, tf_o, nt_o, tie = oracle.render(P, op, pixels=pix)
    sel = (pix[:, 1], pix[:, 0])
    compare_images(color[sel], tf[sel], col_o, tf_o, tie, nt[sel], nt_o, label="10M 4K fused step bands")
    tg = sc.targets[0].numpy()[sel]
    _, G = oracle.loss_l1(col_o.astype(np.float32), tg)
    G = G * (len(pix) / float(W * H))    # the band pixels' share of the full-image mean
    g2o = oracle.raster_backward(P, G.reshape(-1, 3), None, op, pixels=pix)
    _check_grads2d(g2, g2o, "10M bands")
    g3o = oracle.project_backward(sc, cam, g2o, op)
    # 3D gradients and Adam on a sample of Gaussians (the update is per scalar)
    rng = np.random.default_rng(10)
    touched = np.nonzero((g2o != 0).any(axis=0))[0]
    idx = np.union1d(rng.choice(sc.n, 200_000, replace=False), touched[:200_000])
    sub = lambda x: x[:, idx]
    g3s = {nm: (v[idx] if v.ndim == 1 else v[:, idx]) for nm, v in g3o.items()}
    _check_grads3d_and_adam(sub(p0), sub(m0), sub(v0), sub(p1), sub(m1), sub(v1), g3s, 1,
                            dict(PL.DEFAULT_LR), "10M", idx=None)
    # the end of step's projection for the (same) next camera, on the updated parameters
    Pn = oracle.project(_scene_with(sc, torch.from_numpy(p1)), cam, op)
    log(f"  next view's records: {compare_projection(st.proj, Pn)}")
    del st, params
    gc.collect()
    torch.cuda.empty_cache()
