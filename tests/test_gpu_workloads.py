"""Parity of the HIP path with the CPU oracle at the sizes of the measured workloads.
GPU only.

* 1M Gaussians, SH3, 1080p (two of its four views) and 10M Gaussians, SH3, skewed
  clusters, 4K: binning bit-exact from identical projected inputs (the oracle's float
  records are loaded into both binnings); images, final transmittance and N_p on bands of
  rows the oracle renders pixel by pixel; screen-space gradients with the loss gradient
  restricted to those rows (so both sides sum the same pixels).
* 20M Gaussians in four depth slabs, 4K (full size): properties that hold at any size --
  the over-composited partial renders equal the unpartitioned render (Splaxel, section 4.2),
  the gradients through the composite equal the unpartitioned gradients, the
  compacted records scatter back to the dense gradients (ByteSplat, section 6.1), and
  the owner-side decoding of all four slabs' records rebuilds them (section 6.2).
* ByteSplat's owner/renderer split at 100K Gaussians, 512x512: four renderers own bands
  of tile rows; each returns compacted records of the Gaussians sent to it and the
  owner's decoded sum equals one unsplit backward.
* The same partitioned recipe at 200K Gaussians: partial renders, composite, composite
  backward and per-slab gradients against the oracle.
"""
import gc
import math

import numpy as np
import pytest
import torch

import oracle
from differentiable_rasterization_amd import binding as B
from differentiable_rasterization_amd import pipeline as PL
from differentiable_rasterization_amd import scenes
from tests.gpu_util import DEV, compare_images, log, oracle_params, oracle_projection, rel_l2

pytestmark = pytest.mark.gpu


def _band(width, y0, rows):
    return np.stack([np.tile(np.arange(width, dtype=np.int32), rows),
                     np.repeat(np.arange(y0, y0 + rows, dtype=np.int32), width)], axis=1).copy()


def _check_binning(P, cam, n, rp):
    tt, keys, ids, ranges = oracle.bin_f32(P.rec[:, :2].astype(np.float32), P.radii, P.dkey, cam.width,
                                           cam.height)
    proj = oracle_projection(P, n)
    bins = PL.Binning(n, cam.width, cam.height, capacity=len(ids), device=DEV, with_keys=True,
                      with_touched=True)
    k = bins.sort(proj, B.camera_from(cam), rp)
    torch.cuda.synchronize()
    assert k == len(ids)
    assert np.array_equal(bins.tile_ranges.cpu().numpy(), ranges)
    assert np.array_equal(bins.tiles_touched.cpu().numpy(), tt)
    assert np.array_equal(bins.ids[:k].cpu().numpy().view(np.uint32), ids)
    assert np.array_equal(bins.keys[:k].cpu().numpy().view(np.uint64), keys)
    del proj, bins
    return k


def _band_parity(sc, view, bands, check_bins=True):
    """Forward on the whole image, compared on bands of rows; backward with the L1
    gradient of those rows only."""
    cam = sc.cameras[view]
    W, H = cam.width, cam.height
    rp = B.make_params(sc.sh_degree)
    op = oracle_params(rp)
    log(f"  oracle projection of {sc.n} Gaussians, view {view}")
    P = oracle.project(sc, cam, op)
    if check_bins:
        k = _check_binning(P, cam, sc.n, rp)
        log(f"  binning bit-exact, K = {k}")
    params = PL.GaussianParams.from_scene(sc, DEV)
    st = PL.TrainStep(params, W, H, DEV, raster=rp)
    c = B.camera_from(cam)
    st.forward(c)
    torch.cuda.synchronize()
    pix = np.concatenate([_band(W, y0, rows) for y0, rows in bands])
    log(f"  oracle render of {len(pix)} pixels")
    col, tf, nt, tie = oracle.render(P, op, pixels=pix)
    gc_ = st.frame.color.cpu().numpy()[pix[:, 1], pix[:, 0]]
    gt_ = st.frame.t_final.cpu().numpy()[pix[:, 1], pix[:, 0]]
    gn_ = st.frame.n_trav.cpu().numpy()[pix[:, 1], pix[:, 0]]
    compare_images(gc_, gt_, col, tf, tie, gn_, nt)
    # backward: L1 gradient of the band pixels (oracle image), zero elsewhere
    target = sc.targets[view].numpy()[pix[:, 1], pix[:, 0]]
    _, G = oracle.loss_l1(col.astype(np.float32), target)
    G = G.astype(np.float32).reshape(-1, 3)
    Gfull = np.zeros((H, W, 3), np.float32)
    Gfull[pix[:, 1], pix[:, 0]] = G
    st.backward(c, dL_dcolor=torch.from_numpy(Gfull).to(DEV), grads3d=False)
    torch.cuda.synchronize()
    log("  oracle backward of the band")
    g2o = oracle.raster_backward(P, G.astype(np.float64), None, op, pixels=pix)
    g2 = st.grads2d.cpu().numpy()
    errs = {oracle.G_FIELDS[f]: rel_l2(g2[f], g2o[f]) for f in range(9)}
    log(f"  grads2d rel-L2 {errs}")
    assert max(errs.values()) <= 1e-3, errs
    del st, params, P
    gc.collect()
    torch.cuda.empty_cache()


def test_1m_1080p_sampled_parity():
    log("1M 1080p")
    sc = scenes.scene_1m_1080p()
    _band_parity(sc, 0, [(500, 48), (100, 8)])
    _band_parity(sc, 2, [(540, 32)], check_bins=False)


def test_10m_4k_skewed_sampled_parity():
    log("10M 4K skewed")
    sc = scenes.scene_skewed_4k()
    # rows through the dense centre of the image and one off-centre band
    _band_parity(sc, 0, [(1072, 8), (300, 4)])


def _partition_run(sc, t_min, G=None):
    """Unpartitioned and partitioned renders of view 0 on the GPU (depth windows in
    gs_project), the composite, and (if G is given) the backward of both with dL/dC = G."""
    cam = sc.cameras[0]
    W, H = cam.width, cam.height
    n_px = W * H
    c = B.camera_from(cam)
    params = PL.GaussianParams.from_scene(sc, DEV)
    out = {}
    st = PL.TrainStep(params, W, H, DEV, raster=B.make_params(sc.sh_degree, t_min=t_min))
    st.forward(c)
    out["full"] = (st.frame.color.clone(), st.frame.t_final.clone())
    if G is not None:
        st.backward(c, dL_dcolor=G, grads3d=False)
        out["full_g2"] = st.grads2d.clone()
    del st
    torch.cuda.empty_cache()
    slabs = []
    for lo, hi in sc.depth_slabs:
        rp = B.make_params(sc.sh_degree, t_min=t_min, depth_lo=lo, depth_hi=hi)
        s = PL.TrainStep(params, W, H, DEV, raster=rp)
        s.forward(c)
        slabs.append(s)
    cs = [s.frame.color for s in slabs]
    ts = [s.frame.t_final for s in slabs]
    comp_c = torch.zeros(H, W, 3, device=DEV)
    comp_t = torch.zeros(H, W, device=DEV)
    B.gs_composite_over(cs, ts, n_px, t_min, comp_c, comp_t)
    out["comp"] = (comp_c, comp_t)
    out["slabs"] = slabs
    if G is not None:
        dcs = [torch.zeros(H, W, 3, device=DEV) for _ in slabs]
        dts = [torch.zeros(H, W, device=DEV) for _ in slabs]
        B.gs_composite_over_bwd(cs, ts, n_px, t_min, G, None, dcs, dts)
        g2 = torch.zeros_like(out["full_g2"])
        for s, dc, dt in zip(slabs, dcs, dts):
            s.backward(c, dL_dcolor=dc, dL_dt=dt, grads3d=False)
            g2 += s.grads2d     # each Gaussian lies in one slab; the others give it zeros
        out["part_g2"] = g2
        out["dcs"], out["dts"] = dcs, dts
    torch.cuda.synchronize()
    return out


def _check_records(g2):
    """ByteSplat section 6: the compacted records are exactly the Gaussians with a
    non-zero field, in ascending order, and scatter back to the dense gradients."""
    n = g2.shape[1]
    records = torch.zeros(n, 10, dtype=torch.int32, device=DEV)
    bitmap = torch.zeros((n + 31) // 32, dtype=torch.int32, device=DEV)
    ws = torch.empty(B.gs_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    R = B.gs_compact_grads(g2, n, 0, records, bitmap, ws)
    dense = g2.cpu().numpy()
    nz = (dense != 0).any(axis=0)
    assert R == int(nz.sum())
    rec = records[:R].cpu().numpy().view(np.uint32)
    idx = rec[:, 0].astype(np.int64)
    assert np.array_equal(idx, np.nonzero(nz)[0])
    assert np.array_equal(rec[:, 1:].view(np.float32).T.view(np.uint32), dense[:, idx].view(np.uint32))
    bits = np.unpackbits(bitmap.cpu().numpy().view(np.uint8), bitorder="little")[:n].astype(bool)
    assert np.array_equal(bits, nz)
    return R, records


def test_20m_4k_partitioned_properties():
    log("20M 4K, 4 depth slabs")
    sc = scenes.scene_partitioned_4k()
    cam = sc.cameras[0]
    H, W = cam.height, cam.width
    # theta_T = 0: the partitions are an exact split, composite == unpartitioned up to fp32
    tgt = sc.targets[0].to(DEV)
    probe = _partition_run(sc, 0.0)
    comp_c, comp_t = probe["comp"]
    G = (torch.sign(comp_c - tgt) / (3 * H * W)).contiguous()
    del probe
    torch.cuda.empty_cache()
    out = _partition_run(sc, 0.0, G)
    fc, ft = out["full"]
    cc, ct = out["comp"]
    dc = float((fc - cc).abs().max())
    dt = float((ft - ct).abs().max())
    log(f"  theta_T = 0: composite vs unpartitioned max |dC| {dc:.2e} |dT| {dt:.2e}")
    assert dc <= 2e-5 and dt <= 2e-5
    e = rel_l2(out["part_g2"].cpu().numpy(), out["full_g2"].cpu().numpy())
    log(f"  gradients through the composite vs unpartitioned rel-L2 {e:.2e}")
    assert e <= 1e-4
    parts = []
    for k, s in enumerate(out["slabs"]):
        R, records = _check_records(s.grads2d)
        log(f"  slab {k}: {R} non-zero records of {s.params.n}")
        parts.append((records, R, 0, None, s.params.n))
    # owner side: every Gaussian lies in one slab, so the decoded sum of the four record
    # sets is exactly the sum of the dense slab gradients
    n = out["part_g2"].shape[1]
    owner = torch.zeros_like(out["part_g2"])
    rejected = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.gs_decode_grads(parts, owner, n, rejected)
    torch.cuda.synchronize()
    assert int(rejected.item()) == 0
    assert torch.equal(owner, out["part_g2"])
    del out, parts, owner
    torch.cuda.empty_cache()
    # theta_T = 1e-4: termination inside a slab differs from the global one by at most
    # theta_T times a colour
    out = _partition_run(sc, 1e-4, G)
    fc, ft = out["full"]
    cc, ct = out["comp"]
    cmax = float(fc.abs().max())
    dc = float((fc - cc).abs().max())
    log(f"  theta_T = 1e-4: composite vs unpartitioned max |dC| {dc:.2e} (bound {1e-4 * max(1.0, cmax):.2e})")
    assert dc <= 1e-4 * max(1.0, cmax) + 2e-5
    _slab_band_parity(sc, out, 1e-4, [(1072, 2), (400, 2)])
    del out
    torch.cuda.empty_cache()


def _slab_band_parity(sc, out, t_min, bands):
    """Each 5M-Gaussian slab of the full-size partitioned render against the oracle on
    bands of rows: the partial image, T_k and N_p, and the slab's screen-space gradients
    for the composite backward's dL/dC_k and dL/dT_k restricted to those rows."""
    cam = sc.cameras[0]
    W, H = cam.width, cam.height
    c = B.camera_from(cam)
    pix = np.concatenate([_band(W, y0, rows) for y0, rows in bands])
    sel = (pix[:, 1], pix[:, 0])
    rows = np.zeros(H, bool)
    for y0, r in bands:
        rows[y0:y0 + r] = True
    rows_d = torch.from_numpy(rows).to(DEV)
    for k, s in enumerate(out["slabs"]):
        lo, hi = sc.depth_slabs[k]
        op = oracle_params(B.make_params(sc.sh_degree, t_min=t_min, depth_lo=lo, depth_hi=hi))
        log(f"  slab {k}: oracle projection of the {sc.n} Gaussians in [{lo:.3f}, {hi:.3f})")
        P = oracle.project(sc, cam, op)
        col, tf, nt, tie = oracle.render(P, op, pixels=pix)
        compare_images(s.frame.color.cpu().numpy()[sel], s.frame.t_final.cpu().numpy()[sel], col, tf, tie,
                       s.frame.n_trav.cpu().numpy()[sel], nt, label=f"20M 4K slab {k} bands")
        dck = out["dcs"][k] * rows_d[:, None, None]
        dtk = out["dts"][k] * rows_d[:, None]
        s.backward(c, dL_dcolor=dck.contiguous(), dL_dt=dtk.contiguous(), grads3d=False)
        torch.cuda.synchronize()
        g2o = oracle.raster_backward(P, dck.cpu().numpy()[sel].astype(np.float64),
                                     dtk.cpu().numpy()[sel].astype(np.float64), op, pixels=pix)
        g2 = s.grads2d.cpu().numpy()
        errs = {oracle.G_FIELDS[f]: rel_l2(g2[f], g2o[f]) for f in range(9)}
        log(f"  slab {k} band grads2d rel-L2 max {max(errs.values()):.2e}")
        assert max(errs.values()) <= 1e-3, errs
        del P
        gc.collect()


def test_partitioned_small_against_oracle():
    log("partitioned recipe at 200K, 960x540")
    sc = scenes.scene_partitioned_4k(n=200_000, width=960, height=540)
    cam = sc.cameras[0]
    H, W = cam.height, cam.width
    t_min = 1e-4
    # oracle: partial renders, composite, composite backward, per-slab gradients
    orc = []
    for lo, hi in sc.depth_slabs:
        rp = B.make_params(sc.sh_degree, t_min=t_min, depth_lo=lo, depth_hi=hi)
        op = oracle_params(rp)
        P = oracle.project(sc, cam, op)
        col, tf, nt, tie = oracle.render(P, op)
        orc.append((P, op, col, tf, nt, tie))
    cs_o = [o[2].astype(np.float32) for o in orc]
    ts_o = [o[3].astype(np.float32) for o in orc]
    comp_o, compt_o = oracle.composite(cs_o, ts_o, float(np.float32(t_min)))
    _, G = oracle.loss_l1(comp_o.astype(np.float32), sc.targets[0].numpy())
    G = G.astype(np.float32).reshape(H, W, 3)
    dcs_o, dts_o = oracle.composite_bwd(cs_o, ts_o, float(np.float32(t_min)), G)
    out = _partition_run(sc, t_min, torch.from_numpy(G).to(DEV))
    tie_any = np.zeros((H, W), bool)
    for k, (P, op, col, tf, nt, tie) in enumerate(orc):
        s = out["slabs"][k]
        compare_images(s.frame.color.cpu().numpy(), s.frame.t_final.cpu().numpy(), col, tf, tie,
                       s.frame.n_trav.cpu().numpy(), nt, label=f"200K slab {k} partial render")
        tie_any |= tie
    comp_c, comp_t = out["comp"]
    compare_images(comp_c.cpu().numpy(), comp_t.cpu().numpy(), comp_o.reshape(H, W, 3), compt_o.reshape(H, W),
                   tie_any)
    for k, (P, op, col, tf, nt, tie) in enumerate(orc):
        # the composite backward on the GPU partials matches the oracle's on its own partials
        assert np.abs(out["dcs"][k].cpu().numpy().reshape(-1, 3) - dcs_o[k])[~tie_any.reshape(-1)].max() <= 1e-5
        dts_g = out["dts"][k].cpu().numpy().reshape(-1)
        assert np.abs(dts_g - dts_o[k])[~tie_any.reshape(-1)].max() <= 1e-4 * max(1.0, np.abs(dts_o[k]).max())
        g2o = oracle.raster_backward(P, dcs_o[k].reshape(H, W, 3), dts_o[k].reshape(H, W), op)
        g2 = out["slabs"][k].grads2d.cpu().numpy()
        errs = {oracle.G_FIELDS[f]: rel_l2(g2[f], g2o[f]) for f in range(9)}
        log(f"  slab {k} grads2d rel-L2 {errs}")
        assert max(errs.values()) <= 1e-3, errs
        _check_records(out["slabs"][k].grads2d)


def test_tile_band_renderers_decode_to_full_gradients():
    """ByteSplat sections 2.2 and 6: each renderer owns a band of tile rows and receives
    the Gaussians whose footprint reaches it; Gaussians that reach a band but add nothing
    there come back with all-zero gradients and are elided.  The owner decodes the four
    record sets (Gaussians on band borders arrive from two or more renderers) and gets
    the gradients of one unsplit backward, up to the fp32 summation order."""
    log("100K 512x512, 4 renderer bands")
    sc = scenes.scene_100k()
    cam = sc.cameras[0]
    W, H = cam.width, cam.height
    c = B.camera_from(cam)
    params = PL.GaussianParams.from_scene(sc, DEV)
    st = PL.TrainStep(params, W, H, DEV)
    st.forward(c)
    st.loss(sc.targets[0].to(DEV))
    G = st.frame.dL_dcolor.clone()
    st.backward(c, dL_dcolor=G, grads3d=False)
    full = st.grads2d.clone()
    n = params.n
    m2 = st.proj.rec[:, :2].cpu().numpy().astype(np.float64)
    radii = st.proj.radii.cpu().numpy()
    vis = (radii > 0).all(axis=1)
    # rows a footprint can reach (one pixel of slack around the bounding box)
    lo, hi = m2[:, 1] - radii[:, 1] - 1, m2[:, 1] + radii[:, 1] + 1
    band_rows = 16 * ((H // 16 + 3) // 4)
    parts, keep, sent_total, recs_total = [], [], 0, 0
    for y0 in range(0, H, band_rows):
        y1 = min(H, y0 + band_rows)
        Gk = torch.zeros_like(G)
        Gk[y0:y1] = G[y0:y1]
        st.backward(c, dL_dcolor=Gk, grads3d=False)
        sent = np.nonzero(vis & (hi >= y0) & (lo < y1))[0]
        outside = np.ones(n, bool)
        outside[sent] = False
        assert not bool(st.grads2d[:, torch.from_numpy(outside).to(DEV)].any())
        idx = torch.from_numpy(sent).to(DEV)
        gpart = st.grads2d[:, idx].contiguous()
        m = len(sent)
        records = torch.zeros(max(m, 1), 10, dtype=torch.int32, device=DEV)
        bitmap = torch.zeros(max((m + 31) // 32, 1), dtype=torch.int32, device=DEV)
        ws = torch.empty(max(B.gs_compact_workspace_bytes(m), 256), dtype=torch.uint8, device=DEV)
        R = B.gs_compact_grads(gpart, m, 0, records, bitmap, ws) if m else 0
        parts.append((records, R, 0, idx.to(torch.int32), m))
        keep.append(gpart)
        sent_total += m
        recs_total += R
        log(f"  rows [{y0}, {y1}): {m} Gaussians sent, {R} non-zero records returned")
    owner = torch.zeros(9, n, device=DEV)
    rejected = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.gs_decode_grads(parts, owner, n, rejected)
    torch.cuda.synchronize()
    assert int(rejected.item()) == 0
    assert recs_total < sent_total
    got, want = owner.cpu().numpy(), full.cpu().numpy()
    errs = {oracle.G_FIELDS[f]: rel_l2(got[f], want[f]) for f in range(9)}
    log(f"  decoded vs unsplit rel-L2 {errs}; {sent_total - recs_total} of {sent_total} records elided")
    assert max(errs.values()) <= 1e-5, errs
    # a Gaussian that no band's pixels touch has no record anywhere and stays zero
    untouched = ~(want != 0).any(axis=0)
    assert not (got[:, untouched] != 0).any()


def test_partitioned_step_matches_unpartitioned():
    """PartitionedStep on the 4-slab recipe at 200K Gaussians, 960x540, theta_T = 0: the
    composite equals the unpartitioned render, the gradient planes each slab owner decodes
    from its records equal the unpartitioned gradients of its Gaussians, and the owners'
    projection backward gives the unpartitioned 3D gradients (Splaxel section 4.2;
    ByteSplat section 6)."""
    log("PartitionedStep, 200K 960x540, 4 slabs")
    sc = scenes.scene_partitioned_4k(n=200_000, width=960, height=540)
    subs = scenes.slab_scenes(sc)
    cam = B.camera_from(sc.cameras[0])
    W, H = sc.cameras[0].width, sc.cameras[0].height
    tgt = sc.targets[0].to(DEV)
    # Gaussian i of slab k is Gaussian idx[k][i] of the whole scene
    M = sc.cameras[0].viewmat.double().reshape(4, 4)
    z = (M[2, :3].unsqueeze(1) * sc.means.double()).sum(0) + M[2, 3]
    idx = [torch.nonzero((z >= lo) & (z < hi)).squeeze(1) for lo, hi in sc.depth_slabs]
    assert sum(len(i) for i in idx) == sc.n
    full = PL.TrainStep(PL.GaussianParams.from_scene(sc, DEV), W, H, DEV, raster=B.make_params(sc.sh_degree, t_min=0.0))
    full.forward(cam)
    full.loss(tgt)
    full.backward(cam)
    g3_full = full.params.grad.clone()
    slabs = [PL.GaussianParams.from_scene(s, DEV) for s in subs]
    ps = PL.PartitionedStep(slabs, [(0.0, math.inf)] * 4, W, H, DEV, t_min=0.0)
    ps.forward(cam)
    ps.loss(tgt)
    torch.cuda.synchronize()
    dc = float((ps.color - full.frame.color).abs().max())
    dt = float((ps.t_final - full.frame.t_final).abs().max())
    log(f"  composite vs unpartitioned max |dC| {dc:.2e} |dT| {dt:.2e}")
    assert dc <= 2e-5 and dt <= 2e-5
    # the same loss gradient on both sides (pixels whose sign flips between the two renders
    # would otherwise differ)
    ps.dL_dcolor.copy_(full.frame.dL_dcolor)
    ps.backward(cam)
    for k, st in enumerate(ps.parts):
        B.gs_project_bwd(st.params.gaussians(), cam, st.raster, ps.owner_g2[k], st.params.param_grads())
    torch.cuda.synchronize()
    g2_full = full.grads2d.cpu()
    g3 = g3_full.cpu()
    for k, st in enumerate(ps.parts):
        assert torch.equal(ps.owner_g2[k][:, :st.params.n], st.grads2d)      # decoding is exact
        e2 = rel_l2(ps.owner_g2[k].cpu().numpy(), g2_full[:, idx[k]].numpy())
        e3 = rel_l2(st.params.grad.cpu().numpy(), g3[:, idx[k]].numpy())
        log(f"  slab {k}: {ps.r[k]} records of {st.params.n}; grads2d rel-L2 {e2:.2e}, 3D grads rel-L2 {e3:.2e}")
        assert e2 <= 1e-4 and e3 <= 1e-4


def test_partitioned_overlapped_step_matches_serial():
    """PartitionedStep.step_overlapped (each slab's calls on a stream of its own, the binning
    without host waits, a step's updates running into the next step, each update projecting
    its slab for the next step) gives the serial step's results bit for bit: the composite,
    the loss, each slab's records, and the parameters and Adam moments after the updates,
    after step 1 (joined) and step 3 (step 2's updates left running into it).  Both equal a
    serial step made of separate calls (gs_project at the start, gs_project_bwd and
    gs_adam_step at the end); 200K Gaussians, 960x540, 4 depth slabs, theta_T = 1e-4."""
    log("PartitionedStep overlapped vs serial, 200K 960x540, 4 slabs, 3 steps")
    sc = scenes.scene_partitioned_4k(n=200_000, width=960, height=540)
    subs = scenes.slab_scenes(sc)
    cam = B.camera_from(sc.cameras[0])
    W, H = sc.cameras[0].width, sc.cameras[0].height
    tgt = sc.targets[0].to(DEV)
    mk = lambda: PL.PartitionedStep([PL.GaussianParams.from_scene(s, DEV) for s in subs], [(0.0, math.inf)] * 4,
                                    W, H, DEV, t_min=1e-4)
    serial, over, sep = mk(), mk(), mk()
    over.forward(cam)   # sizes each slab's lists (the overlapped binning does not grow them)
    for st in over.parts:
        st.bins._alloc(int(st.bins.capacity * 1.3) + 4096)
    for step in range(3):
        sep.forward(cam)
        sep.loss(tgt)
        sep.backward(cam)
        for k in range(len(sep.parts)):
            sep.update_part_separate(k, cam)
        serial.step(cam, tgt, next_cam=cam, projected=step > 0)
        over.step_overlapped(cam, tgt, join=step != 1, next_cam=cam, projected=step > 0)   # step 1 runs into 2
        if step == 1:
            continue   # compared after step 2, which is ordered after them
        torch.cuda.synchronize()
        assert over.check_capacity()
        for other in (over, sep):
            assert torch.equal(serial.color, other.color) and torch.equal(serial.t_final, other.t_final)
            assert torch.equal(serial.loss_value, other.loss_value)
            assert serial.r == other.r
            for a, b in zip(serial.parts, other.parts):
                assert torch.equal(a.params.data, b.params.data)
                assert torch.equal(a.params.m, b.params.m) and torch.equal(a.params.v, b.params.v)
            for a, b in zip(serial.owner_g2, other.owner_g2):
                assert torch.equal(a, b)
        log(f"  step {step}: equal; records {over.r}")
