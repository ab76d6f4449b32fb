"""Benchmark of the one-GPU 3D Gaussian splatting training step on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1m|100k|10m] [--no-cpu-baseline]

A step is one training iteration on one view: gs_project -> gs_bin_sort ->
gs_raster_fwd -> gs_loss_l1 -> gs_raster_bwd -> gs_project_bwd -> gs_adam_step,
on seeded synthetic data already resident in HBM.  The default workload is 1M
Gaussians (SH degree 3, 64 clusters in a 20 m cube) at 1920x1080 with four
cameras on a sphere of radius 25; steps cycle through the four views.

Prints one JSON line: value = Gaussian-pixel intersections (sum over pixels of the
number of list entries each pixel composites, N_p of Eq. 1 in ByteSplat section 2.1)
per second of whole training step; ms_per_step = train-step milliseconds.  Per-kernel
times come from HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gaussian-pixel intersections/s (fwd+bwd); train-step ms at 1M Gaussians 1080p"
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3          # published MI355X vector fp32 (packed FMA)
FP32_NONPACKED_TFLOPS = 78.6             # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz

# Algorithmic floating-point work per Gaussian-pixel evaluation (a fused multiply-add
# counts 2, exp2 / reciprocal 1), from the operations of Eq. 1 and Eq. 3:
#  forward  : dx, dy (2); exponent a dx^2 + b dx dy + c dy^2 + log2 o (8); exp2 (1);
#             clamp (1); alpha-check (1); w = T alpha (1); C += w c (6); T *= 1 - alpha (2)
#  backward : forward's exponent, exp2, clamp, check (13); T recovery (2); w (1);
#             colour grads (6); dL/dalpha (3 sub + 3 fma + 1 mul = 10); dpower (1);
#             opacity grad (2); conic / mean moment sums (5); B update (9)
FWD_FLOP_PER_ISECT = 22
BWD_FLOP_PER_ISECT = 49


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="1m", choices=["1m", "100k", "10m", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=96, help="image rows the oracle baseline composites")
    return ap.parse_args()


def make_scene(name):
    from differentiable_rasterization_amd import scenes
    if name == "1m":
        return scenes.scene_1m_1080p(), "1M Gaussians SH3, 64 clusters in a 20 m cube, 1920x1080, 4 views on a r=25 sphere"
    if name == "100k":
        return scenes.scene_100k(), "100K Gaussians SH3, U[-5,5]^3, 512x512, 1 view"
    if name == "10m":
        return scenes.scene_skewed_4k(), "10M Gaussians SH3, 256 skewed anisotropic clusters, 3840x2160, 1 view"
    return scenes.scene_tiny(), "1K Gaussians SH0, 64x64, 1 view"


def hbm_bytes(kernel, n, n_vis, k_sh, n_isect, n_px):
    """Algorithmic HBM bytes per launch (what the method must move at least)."""
    sh = 12 * k_sh
    if kernel == "project":
        return n_vis * (48 + sh + 48) + (n - n_vis) * (12 + 12)    # params read + record written
    if kernel == "project_bwd":
        return n_vis * (48 + sh + 36 + 48 + sh) + (n - n_vis) * (48 + sh)
    if kernel == "adam":
        return n * (11 + 3 * k_sh) * 28                             # p, g, m, v read; p, m, v written
    if kernel == "loss":
        return n_px * 36
    if kernel == "bin_sort":
        return 8 * n + 24 * n_vis + 44 * n_isect
    return None


def cpu_baseline(scene, rows):
    """The oracle, single-threaded, on a bounded sample of view 0: projection of every
    Gaussian, compositing and backward of `rows` image rows, projection backward."""
    import numpy as np
    import oracle
    cam = scene.cameras[0]
    t0 = time.perf_counter()
    P = oracle.project(scene, cam)
    W = cam.width
    y0 = (cam.height - rows) // 2
    pix = np.stack([np.tile(np.arange(W, dtype=np.int32), rows),
                    np.repeat(np.arange(y0, y0 + rows, dtype=np.int32), W)], 1)
    col, tf, nt, tie = oracle.render(P, pixels=pix)
    _, G = oracle.loss_l1(col.astype(np.float32), scene.targets[0].numpy()[y0:y0 + rows].reshape(-1, 3))
    g2 = oracle.raster_backward(P, G.reshape(-1, 3), None, pixels=pix)
    oracle.project_backward(scene, cam, g2)
    dt = time.perf_counter() - t0
    isect = int(nt.sum())
    return {"value": isect / dt, "unit": "Gaussian-pixel intersections/s", "cores": 1, "kind": "oracle",
            "sample": f"view 0: projection + projection backward of all {scene.n} Gaussians, compositing and "
                      f"compositing backward of {rows} rows x {W} px ({isect} intersections) in {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from differentiable_rasterization_amd import binding as B
    from differentiable_rasterization_amd import pipeline as PL

    dev = "cuda"
    scene, desc = make_scene(args.workload)
    cams = [B.camera_from(c) for c in scene.cameras]
    targets = [t.to(dev) for t in scene.targets]
    nviews = len(cams)
    W, H = scene.cameras[0].width, scene.cameras[0].height
    params = PL.GaussianParams.from_scene(scene, dev)
    st = PL.TrainStep(params, W, H, dev)
    # size the intersection lists for every view before timing
    for c in cams:
        st.forward(c)
    st.bins._alloc(int(st.bins.capacity * 1.3) + 4096)
    torch.cuda.synchronize()

    names = ["project", "bin_sort", "raster_fwd", "loss", "raster_bwd", "project_bwd", "adam"]

    def one_step(i, ev=None):
        c, t = cams[i % nviews], targets[i % nviews]
        rec = (lambda k: ev[k].record()) if ev is not None else (lambda k: None)
        rec(0)
        B.gs_project(params.gaussians(), c, st.raster, st.proj.abi())
        rec(1)
        st.bins.sort(st.proj, c, st.raster)
        rec(2)
        f = st.frame
        B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), c, st.raster, f.color, f.t_final, f.n_trav, f.n_trav_sum)
        rec(3)
        B.gs_loss_l1(f.color, t, f.n_px, f.loss, f.dL_dcolor, f.loss_ws)
        rec(4)
        st.backward_raster(c)
        rec(5)
        st.backward_project(c)
        rec(6)
        st.adam()
        rec(7)

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    st.frame.n_trav_sum.zero_()
    k_isect = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, events[i])
        k_isect.append(st.bins.n_isect)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    isect_total = int(st.frame.n_trav_sum.item())
    per_kernel = {nm: sum(events[s][j].elapsed_time(events[s][j + 1]) for s in range(args.steps)) / args.steps
                  for j, nm in enumerate(names)}
    ms_step = wall * 1e3 / args.steps
    isect_step = isect_total / args.steps
    n = scene.n
    n_vis = int((st.proj.radii[:, 0] > 0).sum().item())
    k_sh = scene.k_sh
    kmean = sum(k_isect) / len(k_isect)
    kernels = {}
    for nm, ms in per_kernel.items():
        entry = {"ms": round(ms, 4)}
        by = hbm_bytes(nm, n, n_vis, k_sh, kmean, W * H)
        if by is not None:
            entry.update(bound="hbm", algorithmic_bytes=int(by), achieved_GBs=round(by / (ms * 1e-3) / 1e9, 1),
                         frac=round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        elif nm in ("raster_fwd", "raster_bwd"):
            fl = (FWD_FLOP_PER_ISECT if nm == "raster_fwd" else BWD_FLOP_PER_ISECT) * isect_step
            tf = fl / (ms * 1e-3) / 1e12
            entry.update(bound="alu", algorithmic_flop=int(fl), achieved_TFLOPs=round(tf, 3),
                         frac=round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                         frac_nonpacked=round(tf / FP32_NONPACKED_TFLOPS, 4),
                         isect_per_s=round(isect_step / (ms * 1e-3), 1))
        kernels[nm] = entry
    dom = max(per_kernel, key=per_kernel.get)
    d = kernels[dom]
    if d.get("bound") == "hbm":
        roof = {"kernel": dom, "bound": "hbm", "achieved": d["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac"], "traffic": None}
    else:
        roof = {"kernel": dom, "bound": "alu", "achieved": d["achieved_TFLOPs"], "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": d["frac"], "traffic": None}
    out = {
        "metric": METRIC, "value": round(isect_total / wall, 1), "unit": "Gaussian-pixel intersections/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": desc, "gaussians": n, "sh_degree": scene.sh_degree, "image": [W, H],
                   "views": nviews, "step": "one view: fwd + L1 + bwd + Adam"},
        "roofline": roof,
        "intersections_per_step": round(isect_step, 1),
        "tile_entries_per_step": round(kmean, 1),
        "visible_gaussians": n_vis,
        "raster_isect_per_s": round(isect_step / ((per_kernel["raster_fwd"] + per_kernel["raster_bwd"]) * 1e-3), 1),
        "kernels": kernels,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(scene, min(args.cpu_rows, H))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
