"""Benchmark of the one-GPU 3D Gaussian splatting training step on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1m|100k|10m|20m|tiny] [--no-cpu-baseline]
                    [--cpu-rows R] [--copy-calibration-mib M] [--batch B]

A step is one training iteration on one view: projection -> gs_bin_sort ->
gs_raster_fused_l1 (forward rasterization, L1 loss and backward rasterization in one
kernel) -> gs_grad_aggregate_adam_project (the per-Gaussian gradient sum, projection
backward, Adam and the projection of the updated Gaussians for the next step's view in
one pass, so each step's projection is done by the step before it; the first step's
records come from gs_project before the warm-up).  --separate-raster runs gs_raster_fwd,
gs_loss_l1 and gs_raster_bwd_partials in place of the fused kernel; --unfused also runs
gs_project at the start of each step and gs_grad_aggregate, gs_project_bwd and
gs_adam_step at its end.  The data are seeded, synthetic and
already resident in HBM.  The default workload is 1M
Gaussians (SH degree 3, 64 clusters in a 20 m cube) at 1920x1080 with four
cameras on a sphere of radius 25; steps cycle through the four views.

Prints one JSON line: value = Gaussian-pixel intersections (sum over pixels of the
number of list entries each pixel composites, N_p of Eq. 1 in ByteSplat section 2.1)
per second of whole training step; ms_per_step = train-step milliseconds.  Per-kernel
times come from HIP events recorded on the stream the kernels run on (timing-only events
without the system-scope fence, see TimingEvent).

--workload 20m measures the partitioned step instead (PartitionedStep): 20M Gaussians at
3840x2160 in four camera-space depth slabs of 5M, each rendered on its own and
over-composited, L1 on the composite, the composite backward, each slab's backward
rasterization and per-Gaussian sum, compaction of its non-zero gradient records, their
decoding into the slab owner's gradient planes, and the owner's projection backward and
Adam in one pass, which also projects the updated slab for the next step (so a step
starts at the binning).  The timed steps run each slab's calls on a stream of its own (the slabs share
nothing between the composites); `kernels` times every call with events in as many
serial steps afterwards, whose wall time is serial_ms_per_step.

--batch B (2..4) measures BatchTrainStep instead: one optimiser step over B views (the
workload's views in turn), each binned and rasterized with the fused forward + L1 +
backward, then one gs_grad_aggregate_adam_batch pass (the views' gradient mean, Adam with
the batch hyper-parameters of the ROCm blog's "Batching and Hyperparameter Scaling", and
the next batch's projections).  ms_per_step is per optimiser step (B views).

roofline: the longer of the backward raster kernel (k_raster_fused_l1 by default,
k_raster_bwd with --separate-raster; bound by VALU arithmetic: FLOP_FWD floating-point
operations per (pixel, record) pair the forward walk evaluates and FLOP_BWD per pair the
backward walk evaluates, with the pairs counted on the device by the fused kernel's
counting instance in an untimed call on each view's lists after the timed steps; peak: the
non-packed fp32 VALU rate) and k_grad_adam (bound by HBM; hbm_bytes), one launch each per
step; roofline_next the other.  roofline.traffic is the HBM traffic of one launch
from the stored counter summary (profiles/), or null if the kernel's sources changed
since those counters were taken.  --copy-calibration-mib runs a plain copy-like kernel of
known size before the timed steps, for the counter runs that normalise FETCH_SIZE and
WRITE_SIZE.  skew: the last step's longest tile list over the mean and the share of the
entries in the longest 1 % of tiles (and at 10M the share of the means inside the dense
central sub-cube of the clustered recipe).  The timed loops run with Python's cyclic
garbage collector off (quiet_gc).
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def quiet_gc():
    """Collects once, then switches Python's cyclic garbage collector off for the timed
    loops, so that no collection pauses the host inside a timed call.  Without the
    collection up front, one pause of tens of milliseconds (with the GPU idle) landed
    inside a single call of the 20M step's per-call breakdown, presumably the collection
    that freed the scene's multi-gigabyte host tensors."""
    gc.collect()
    gc.disable()


METRIC = "Gaussian-pixel intersections/s (fwd+bwd); train-step ms at 1M Gaussians 1080p"
METRIC_OF = {"1m": METRIC,
             "100k": "Gaussian-pixel intersections/s (fwd+bwd); train-step ms at 100K Gaussians 512x512",
             "10m": "Gaussian-pixel intersections/s (fwd+bwd); train-step ms at 10M Gaussians 4K (skewed)",
             "20m": "Gaussian-pixel intersections/s (fwd+bwd); train-step ms at 20M Gaussians 4K in 4 depth slabs",
             "tiny": "Gaussian-pixel intersections/s (fwd+bwd); train-step ms at 1K Gaussians 64x64"}
HBM_PEAK_GBS = 8000.0
# fp32 VALU peak reachable without packed-FP32 instructions (the build excludes them):
# 256 CU x 4 SIMD x 16 lanes x 2 flop (FMA) x 2.4 GHz; the published 157.3 needs packed FMA
FP32_VALU_PEAK_TFLOPS = 78.6
FP32_PACKED_PUBLISHED_TFLOPS = 157.3

# Algorithmic floating-point work per evaluated (pixel, record) pair, from the operation
# lists of ByteSplat Eq. 1 (forward: offset, quadratic form, exp, clamp and alpha-check,
# blend, transmittance update: 26 flop + 1 exp) and Eq. 3 / Eq. 4 (backward: the forward's
# alpha, T recovery, colour and alpha gradients, colour-behind update, power / conic / mean /
# opacity gradients and their per-Gaussian sums: 61 flop + 1 exp + 1 reciprocal).  Every
# record a quadrant wave walks is evaluated for all 64 of its lanes (branch-free), so the
# pairs are 64 x the records walked, counted on the device (gs_raster_fused_l1 walk_counts).
FLOP_FWD, FLOP_BWD = 27, 63
ALU_KERNELS = ("raster_fwd", "raster_bwd", "raster_fused")


def alu_flop(nm, walk):
    """Algorithmic flop of one launch of raster kernel nm; walk = per-launch (forward
    records, backward records, accepted pairs) of the quadrant waves."""
    pf, pb = 64.0 * walk[0], 64.0 * walk[1]
    return {"raster_fwd": FLOP_FWD * pf, "raster_bwd": FLOP_BWD * pb,
            "raster_fused": FLOP_FWD * pf + FLOP_BWD * pb}[nm]


def alu_entry(nm, ms, walk, isect):
    fl = alu_flop(nm, walk)
    tf = fl / (ms * 1e-3) / 1e12
    return dict(bound="alu", algorithmic_flop=int(fl), achieved_TFLOPs=round(tf, 3),
                frac=round(tf / FP32_VALU_PEAK_TFLOPS, 4), isect_per_s=round(isect / (ms * 1e-3), 1))


def alu_roofline(kern, nm, d, walk, isect, traffic):
    return {"kernel": kern, "bound": "alu", "achieved": d["achieved_TFLOPs"], "peak": FP32_VALU_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": d["frac"], "traffic": traffic,
            "flop_per_pair": {"fwd": FLOP_FWD if nm != "raster_bwd" else 0, "bwd": FLOP_BWD if nm != "raster_fwd" else 0},
            "pairs_per_launch": {"fwd_evaluated": round(64.0 * walk[0], 1) if nm != "raster_bwd" else 0,
                                 "bwd_evaluated": round(64.0 * walk[1], 1) if nm != "raster_fwd" else 0,
                                 "fwd_accepted": round(walk[2], 1), "sum_n_p": round(isect, 1)},
            "launch_ms": d["ms"], "peak_packed_published": FP32_PACKED_PUBLISHED_TFLOPS}


def count_walks(runs):
    """runs: (callable(walk_counts)) per launch to count; each runs the fused kernel's counting
    instance once.  Returns the (forward records, backward records, accepted pairs) of each."""
    import torch
    out = []
    for run in runs:
        wc = torch.zeros(3, dtype=torch.int64, device="cuda")
        run(wc)
        out.append([int(x) for x in wc.cpu()])
    return out
# stored counter traffic of the kernels that can dominate the step (1M / 1080p workload)
TRAFFIC_SUMMARY = {"k_grad_adam_batch": os.path.join(ROOT, "profiles", "k_grad_adam_batch_1m_1080p_traffic.txt"),
                   "k_raster_bwd": os.path.join(ROOT, "profiles", "k_raster_bwd_1m_1080p_traffic.txt"),
                   "k_raster_fused_l1": os.path.join(ROOT, "profiles", "k_raster_fused_l1_1m_1080p_traffic.txt"),
                   "k_grad_adam": os.path.join(ROOT, "profiles", "k_grad_adam_1m_1080p_traffic.txt")}
KERNEL_OF = {"raster_bwd": "k_raster_bwd", "grad_adam": "k_grad_adam", "grad_adam_project": "k_grad_adam",
             "raster_fused": "k_raster_fused_l1"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="1m", choices=["1m", "100k", "10m", "20m", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1080, help="image rows the oracle baseline composites")
    ap.add_argument("--unfused", action="store_true",
                    help="separate gs_grad_aggregate, gs_project_bwd and gs_adam_step calls instead of the fused pass")
    ap.add_argument("--separate-raster", action="store_true",
                    help="gs_raster_fwd, gs_loss_l1 and gs_raster_bwd_partials instead of gs_raster_fused_l1")
    ap.add_argument("--binning-launch", choices=["auto", "graph", "eager"], default="auto",
                    help="replay the binning's per-view HIP graph, launch its kernels one by one, or (auto) time a few "
                         "untimed steps each way after the warm-up and keep the faster")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the untimed pass that times every call separately")
    ap.add_argument("--batch", type=int, default=1, help="views per optimiser step (BatchTrainStep for 2..4)")
    ap.add_argument("--serial-views", action="store_true",
                    help="with --batch: bin and rasterize the views one after another on one stream instead of one "
                         "stream per view")
    ap.add_argument("--loss", choices=["l1", "l1_dssim"], default="l1",
                    help="l1_dssim: (1 - lambda) L1 + lambda (1 - SSIM)/2 with lambda 0.2 (gs_loss_l1_dssim) between "
                         "the separate forward and backward raster calls")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a copy-like kernel over this many MiB before timing (counter normalisation)")
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
    if kernel == "grad_aggregate":
        return 36 * n_isect + 36 * n                                # one partial per (tile, Gaussian); grads2d
    if kernel == "grad_adam":                                       # partials; p, m, v read and written
        return 36 * n_isect + n * (11 + 3 * k_sh) * 24
    if kernel == "grad_adam_project":                               # the same + the next view's projection
        return 36 * n_isect + n * (11 + 3 * k_sh) * 24 + n_vis * 60 + (n - n_vis) * 12
    if kernel == "update":                                          # grads2d read; p, m, v; the next projection
        return 36 * n + n * (11 + 3 * k_sh) * 24 + n_vis * 60 + (n - n_vis) * 12
    return None


def partition_bytes(kernel, parts, n_px, n, records):
    """Algorithmic HBM bytes per call of the partitioned step's own kernels."""
    if kernel == "composite":          # C_k, T_k read; C, T written
        return (16 * parts + 16) * n_px
    if kernel == "composite_bwd":      # C_k, T_k and dL/dC read; dL/dC_k, dL/dT_k written
        return (32 * parts + 12) * n_px
    if kernel == "compact":            # grads2d read, records and the bitmap written
        return 36 * n + 40 * records + n // 8
    if kernel == "decode":             # records read; 9 fields read and written (zeroing: 36 B per Gaussian)
        return 40 * records + 72 * records + 36 * n
    return None


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    skips the system-scope release fence (a cache writeback and invalidation) that a
    default event performs, which costs the stream several microseconds per record on this
    GPU.  Recorded on the current (torch) stream, the stream the kernels are launched on.
    Uses the HIP runtime torch has loaded."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            import torch
            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        rc = self._lib().hipEventRecord(self.ev, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        rc = self._lib().hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(scene, rows):
    """The oracle, single-threaded, on a bounded sample of view 0: projection of every
    Gaussian, compositing and backward of `rows` image rows, projection backward.  Runs
    pinned to one host core (os.sched_setaffinity of this thread, restored afterwards),
    before the GPU is used."""
    import numpy as np
    import oracle
    cam = scene.cameras[0]
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})
    try:
        out = _cpu_baseline_pinned(scene, rows, oracle, np, cam)
    finally:
        os.sched_setaffinity(0, set(allowed))
    out.update(pinned_core=core, cpu_model=cpu_model())
    return out


def _cpu_baseline_pinned(scene, rows, oracle, np, cam):
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


def _band_worker(args):
    """One process of the parallel oracle leg: compositing and compositing backward of a
    band of rows (the projection is inherited from the parent)."""
    import numpy as np
    import oracle
    ys, W = args
    P, target = _PAR_STATE["P"], _PAR_STATE["target"]
    ys = np.asarray(ys, dtype=np.int32)
    pix = np.stack([np.tile(np.arange(W, dtype=np.int32), len(ys)), np.repeat(ys, W)], 1)
    col, tf, nt, tie = oracle.render(P, pixels=pix)
    _, G = oracle.loss_l1(col.astype(np.float32), target[ys].reshape(-1, 3))
    oracle.raster_backward(P, G.reshape(-1, 3), None, pixels=pix)
    return int(nt.sum())


_PAR_STATE = {}


def cpu_baseline_parallel(scene, rows):
    """The same per-pixel work as cpu_baseline (compositing and its backward of `rows`
    rows of view 0), the rows dealt round-robin to P forked processes (P = the CPU share,
    at most 16), the projection done once beforehand and not timed.  Runs before the GPU
    is used."""
    import multiprocessing as mp
    import oracle
    cam = scene.cameras[0]
    procs = max(1, min(16, len(os.sched_getaffinity(0))))
    _PAR_STATE["P"] = oracle.project(scene, cam)
    _PAR_STATE["target"] = scene.targets[0].numpy()
    y0 = (cam.height - rows) // 2
    bands = [(list(range(y0 + b, y0 + rows, procs)), cam.width) for b in range(min(procs, rows))]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(bands)) as pool:
        isect = sum(pool.map(_band_worker, bands))
    dt = time.perf_counter() - t0
    _PAR_STATE.clear()
    return {"value": isect / dt, "unit": "Gaussian-pixel intersections/s", "cores": len(bands), "kind": "oracle",
            "sample": f"view 0: compositing and compositing backward of {rows} rows x {cam.width} px "
                      f"({isect} intersections), rows dealt round-robin to {len(bands)} processes, in {dt:.2f} s "
                      "(projection not timed)", "cpu_model": cpu_model()}


def device_info():
    import torch
    info = {"name": torch.cuda.get_device_name(0), "hip": getattr(torch.version, "hip", None)}
    try:
        pr = torch.cuda.get_device_properties(0)
        info["compute_units"] = pr.multi_processor_count
        info["arch"] = getattr(pr, "gcnArchName", None)
    except Exception:
        pass
    try:   # current shader clock from the driver's DPM table, where readable
        import glob
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            cur = [ln for ln in open(f).read().splitlines() if ln.strip().endswith("*")]
            if cur:
                info["sclk"] = cur[0].split(":", 1)[1].strip(" *")
                break
    except Exception:
        pass
    return info


def choose_binning_launch(one_step, use_graph, step0, n, slots):
    """Runs n untimed training steps with the binning replayed as graphs and n with its
    kernels launched one by one, twice each, and keeps the faster way in use_graph[0].
    Which is faster depends on the host: a graph replay costs the GPU a few microseconds
    more, eager launches cost the host ~30 launches per binning.  The steps are ordinary
    training steps (step0, step0 + 1, ...); eager steps queue the sort without a host wait.
    Returns the wall ms per step of each run and the number of steps taken ("steps")."""
    import torch
    counts = torch.zeros(slots, 2, dtype=torch.int64, device="cuda")
    per = {"graph": [], "eager": []}
    i = step0
    for _ in range(2):
        for mode in ("graph", "eager"):
            use_graph[0] = mode == "graph"
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(n):
                one_step(i, counts=counts if slots > 1 else counts[0])
                i += 1
            torch.cuda.synchronize()
            per[mode].append(round((time.perf_counter() - t) * 1e3 / n, 4))
    use_graph[0] = min(per["graph"]) <= min(per["eager"])
    return {**per, "steps": i - step0}


class CallTimer:
    """Timing events around calls, summed by name after a synchronisation.  The events come
    from a pool created up front (n_events of them), so that no event is created between
    the calls being timed: creating HIP events inside a timed loop left one-time host stalls
    of tens of ms in the partitioned step's trace, with the GPU idle.  `created_late` counts
    events the pool could not supply."""

    def __init__(self, n_events=0):
        self.marks = []
        self.pool = [TimingEvent() for _ in range(n_events)]
        self.created_late = 0

    def _event(self):
        if self.pool:
            return self.pool.pop()
        self.created_late += 1
        return TimingEvent()

    def __call__(self, name):
        timer = self

        class _Ctx:
            def __enter__(self):
                self.a = timer._event()
                self.a.record()

            def __exit__(self, *exc):
                b = timer._event()
                b.record()
                timer.marks.append((name, self.a, b))
        return _Ctx()

    def totals(self):
        out = {}
        for name, a, b in self.marks:
            out[name] = out.get(name, 0.0) + a.elapsed_time(b)
        return out


def main_partitioned(args):
    """The partitioned step of --workload 20m (see the module docstring)."""
    import math
    import torch
    from differentiable_rasterization_amd import binding as B
    from differentiable_rasterization_amd import pipeline as PL
    from differentiable_rasterization_amd import scenes

    dev = "cuda"
    scene = scenes.scene_partitioned_4k()
    desc = "20M Gaussians SH3, 256 skewed anisotropic clusters, 3840x2160, 1 view, 4 depth slabs of 5M"
    subs = scenes.slab_scenes(scene)
    cam = B.camera_from(scene.cameras[0])
    target = scene.targets[0].to(dev)
    W, H = scene.cameras[0].width, scene.cameras[0].height
    slabs = [PL.GaussianParams.from_scene(s, dev) for s in subs]
    del subs
    # the slabs are disjoint and depth-ordered, so each projects without a depth window
    ps = PL.PartitionedStep(slabs, [(0.0, math.inf)] * len(slabs), W, H, dev, t_min=1e-4)
    ps.forward(cam)
    for st in ps.parts:
        st.bins._alloc(int(st.bins.capacity * 1.3) + 4096)
    torch.cuda.synchronize()

    # Each slab's update (projection backward + Adam) also projects the updated slab for the
    # next step's camera, so a step after the first starts at the binning.
    def one_step(t):
        for k, st in enumerate(ps.parts):
            with t("bin_sort"):
                st.bins.sort(st.proj, cam, st.raster)
            with t("raster_fwd"):
                f = st.frame
                B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), cam, st.raster, f.color, f.t_final, f.n_trav,
                                f.n_trav_sum)
        with t("composite"):
            ps.composite()
        with t("loss"):
            ps.loss(target)
        with t("composite_bwd"):
            ps.composite_backward()
        for k, st in enumerate(ps.parts):
            with t("raster_bwd"):
                st.backward_partials(cam, dL_dcolor=ps.dcs[k], dL_dt=ps.dts[k])
            with t("grad_aggregate"):
                B.gs_grad_aggregate(st.params.gaussians(), st.proj.abi(), st.bins.abi(), cam, st.raster,
                                    st.grads2d, None)
            with t("compact"):
                ps.compact_part(k)
            with t("decode"):
                ps.decode_part(k)
            with t("update"):
                ps.update_part(k, cam, next_cam=cam)

    # The timed steps run the slabs side by side (PartitionedStep.step_overlapped: each slab
    # on a stream of its own, binning without host waits); the per-call breakdown comes from
    # the same number of serial steps afterwards, every call between HIP events (events
    # around overlapped calls would not time the calls).
    tgt = target
    quiet_gc()
    for _ in range(args.warmup):   # ps.forward above projected every slab for cam
        ps.step_overlapped(cam, tgt, join=False, next_cam=cam, projected=True)
    ps.join()
    torch.cuda.synchronize()
    if not ps.check_capacity():
        raise RuntimeError("a slab's lists outgrew their buffers during the warm-up; rerun")
    for st in ps.parts:
        st.frame.n_trav_sum.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        # a slab's update overlaps the next step's binning of the others
        ps.step_overlapped(cam, tgt, join=False, next_cam=cam, projected=True)
    ps.join()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not ps.check_capacity():
        raise RuntimeError("a slab's lists outgrew their buffers during the timed steps; rerun")
    isect_step = sum(int(st.frame.n_trav_sum.item()) for st in ps.parts) / args.steps
    probe = CallTimer()
    one_step(probe)   # one untimed serial step, to count the calls of a step
    torch.cuda.synchronize()
    timer = CallTimer(2 * len(probe.marks) * args.steps)
    torch.cuda.synchronize()
    ts0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(timer)
    torch.cuda.synchronize()
    serial_wall = time.perf_counter() - ts0
    per_kernel = {nm: ms / args.steps for nm, ms in timer.totals().items()}
    # the raster walks of the last step's slab lists, counted by the fused kernel's counting
    # instance (its forward and backward walks are those of the separate raster kernels;
    # the target only sets dL/dC, which does not change which records are walked)
    walks = count_walks([lambda wc, st=st: st.fused_l1(cam, st.frame.color.clone(), walk_counts=wc)
                         for st in ps.parts])
    walk_step = [sum(w[j] for w in walks) for j in range(3)]
    parts = len(ps.parts)
    n = sum(st.params.n for st in ps.parts)
    n_vis = sum(int((st.proj.radii[:, 0] > 0).sum().item()) for st in ps.parts)
    k_isect = sum(st.bins.n_isect for st in ps.parts)
    records = sum(ps.r)
    k_sh = scene.k_sh
    kernels = {}
    for nm, ms in per_kernel.items():
        entry = {"ms": round(ms, 4)}
        by = partition_bytes(nm, parts, W * H, n, records)
        if by is None:
            by = hbm_bytes(nm, n, n_vis, k_sh, k_isect, W * H)
        if by is not None:
            entry.update(bound="hbm", algorithmic_bytes=int(by), achieved_GBs=round(by / (ms * 1e-3) / 1e9, 1),
                         frac=round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        elif nm in ALU_KERNELS:
            entry.update(alu_entry(nm, ms, walk_step, isect_step))
        kernels[nm] = entry
    dom = max(per_kernel, key=per_kernel.get)
    d = kernels[dom]
    kern = {"raster_bwd": "k_raster_bwd", "raster_fwd": "k_raster_fwd", "bin_sort": "gs_bin_sort",
            "update": "k_proj_bwd_adam"}.get(dom, dom)
    if d.get("bound") == "alu":
        per_launch = dict(d, ms=round(d["ms"] / parts, 4))
        roof = alu_roofline(kern, dom, per_launch, [w / parts for w in walk_step], isect_step / parts, None)
    else:
        roof = {"kernel": kern, "bound": "hbm", "achieved": d["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac"], "traffic": None, "algorithmic_bytes": d["algorithmic_bytes"],
                "launch_ms": d["ms"]}
    out = {
        "metric": METRIC_OF["20m"], "value": round(isect_step * args.steps / wall, 1),
        "unit": "Gaussian-pixel intersections/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": desc, "gaussians": n, "sh_degree": scene.sh_degree, "image": [W, H], "views": 1,
                   "slabs": parts, "slab_gaussians": [st.params.n for st in ps.parts],
                   "step": "per slab binning + forward; composite; L1; composite backward; per slab backward "
                           "raster + per-Gaussian sum + compaction + decoding + projection backward + Adam + the "
                           "next step's projection (the last three in one pass)",
                   "schedule": "each slab's calls on a stream of its own (PartitionedStep.step_overlapped)"},
        "roofline": roof,
        "intersections_per_step": round(isect_step, 1),
        "tile_entries_per_step": k_isect,
        "records_per_step": records,
        "visible_gaussians": n_vis,
        "serial_ms_per_step": round(serial_wall * 1e3 / args.steps, 4),
        "kernels_note": "every call timed with events in as many serial steps after the timed ones; summed over "
                        "the slabs",
        "breakdown_events_created_late": timer.created_late,
        "kernels": kernels,
        "device": torch.cuda.get_device_name(0),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main_batch(args):
    """--batch B: BatchTrainStep over the workload's views (see the module docstring)."""
    import torch
    from differentiable_rasterization_amd import binding as B
    from differentiable_rasterization_amd import pipeline as PL

    dev = "cuda"
    scene, desc = make_scene(args.workload)
    cams = [B.camera_from(c) for c in scene.cameras]
    targets = [t.to(dev) for t in scene.targets]
    nviews = len(cams)
    W, H = scene.cameras[0].width, scene.cameras[0].height
    bs = args.batch
    params = PL.GaussianParams.from_scene(scene, dev)
    bt = PL.BatchTrainStep(params, W, H, bs, dev)
    views_of = lambda i: [(i * bs + k) % nviews for k in range(bs)]
    # size every view's lists before timing
    for v in range(nviews):
        bt.project([cams[v]] * bs)
        for k in range(bs):
            bt.sort(k, cams[v])
    for b in bt.bins:
        b._alloc(int(b.capacity * 1.3) + 4096)
    torch.cuda.synchronize()
    # each (batch slot, view) pair's binning as a HIP graph; each replay adds its counts to acc
    acc = torch.zeros(2, dtype=torch.int64, device=dev)
    graphs = None
    if args.binning_launch != "eager":
        pairs = sorted({(k, v) for i in range(nviews) for k, v in enumerate(views_of(i))})
        pair_counts = torch.zeros(len(pairs), 2, dtype=torch.int64, device=dev)
        graphs = {(k, v): PL.BinSortGraph(bt.bins[k], bt.proj[k], cams[v], bt.raster, pair_counts[j], acc)
                  for j, (k, v) in enumerate(pairs)}
    use_graph = [graphs is not None]

    vstreams = None if args.serial_views else PL.ViewStreams(bs)

    def one_step(i, ev=None, counts=None):
        """Each view's binning and rasterization on its own stream (vstreams), the update on
        the current stream after them; ev[2k], ev[2k + 1] bracket view k's rasterization on
        the stream it runs on."""
        vs, nv = views_of(i), views_of(i + 1)
        rec = (lambda k: ev[k].record()) if ev is not None else (lambda k: None)
        if vstreams is not None:
            vstreams.fork()
        for k, v in enumerate(vs):
            with (torch.cuda.stream(vstreams.streams[k]) if vstreams is not None else contextlib.nullcontext()):
                if use_graph[0]:
                    graphs[(k, v)].replay()
                elif counts is None:
                    bt.sort(k, cams[v])
                else:
                    bt.bins[k].sort_async(bt.proj[k], cams[v], bt.raster, counts[k])
                rec(2 * k)
                bt.render(k, cams[v], targets[v])
                rec(2 * k + 1)
        if vstreams is not None:
            vstreams.join()
        rec(2 * bs)
        bt.update([cams[v] for v in vs], [cams[v] for v in nv])
        rec(2 * bs + 1)

    if args.copy_calibration_mib > 0:
        # a copy-like kernel of known size (reads and writes M MiB) for counter normalisation
        src = torch.ones(args.copy_calibration_mib << 18, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    bt.project([cams[v] for v in views_of(0)])
    quiet_gc()
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    step0 = args.warmup
    launch_trials = None
    if args.binning_launch == "auto":
        launch_trials = choose_binning_launch(one_step, use_graph, step0, 4, bs)
        step0 += launch_trials.pop("steps")
    for f in bt.frame:
        f.n_trav_sum.zero_()
    events = [[TimingEvent() for _ in range(2 * bs + 2)] for _ in range(args.steps)]
    counts = torch.zeros(args.steps, bs, 2, dtype=torch.int64, device=dev)
    acc.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(step0 + i, events[i], counts[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if use_graph[0]:
        k_sum, need = (int(x) for x in acc.cpu())
        if need != 0:
            raise RuntimeError("intersection lists overflowed during the timed steps")
        k_mean = k_sum / (args.steps * bs)
    else:
        cnt = counts.cpu()
        if int(cnt[:, :, 1].max()) != 0:
            raise RuntimeError("intersection lists overflowed during the timed steps")
        k_mean = float(cnt[:, :, 0].double().mean())
    raster_ms = sum(events[s][2 * k].elapsed_time(events[s][2 * k + 1]) for s in range(args.steps)
                    for k in range(bs)) / (args.steps * bs)
    update_ms = sum(events[s][2 * bs].elapsed_time(events[s][2 * bs + 1]) for s in range(args.steps)) / args.steps
    isect_total = sum(int(f.n_trav_sum.item()) for f in bt.frame)
    isect_view = isect_total / (args.steps * bs)
    n = scene.n
    n_vis = int((bt.proj[0].radii[:, 0] > 0).sum().item())
    by = 36 * k_mean * bs + n * (11 + 3 * scene.k_sh) * 24 + bs * (n_vis * 96 + (n - n_vis) * 12)
    # the walks of each batch slot's last lists, counted by the fused kernel's counting instance
    last_views = views_of(step0 + args.steps - 1)   # the views whose lists the bins hold now
    walks = count_walks([lambda wc, k=k: B.gs_raster_fused_l1(
        bt.params.gaussians(), bt.bins[k].abi(), cams[last_views[k]], bt.raster, targets[last_views[k]],
        bt.frame[k].color, bt.frame[k].t_final, bt.frame[k].n_trav, None, None, bt.frame[k].fused_ws,
        walk_counts=wc) for k in range(bs)])
    walk_view = [sum(w[j] for w in walks) / bs for j in range(3)]
    fl = alu_flop("raster_fused", walk_view)
    if vstreams is None:
        raster_entry = dict(ms=round(raster_ms, 4), **alu_entry("raster_fused", raster_ms, walk_view, isect_view),
                            note="per view")
    else:   # the views overlap: the window on a view's stream is not the kernel's duration
        raster_entry = {"window_ms": round(raster_ms, 4), "bound": "alu", "algorithmic_flop": int(fl),
                        "note": "per view; window between events on the view's stream while the other views' "
                                "binning and rasterization run beside it (not a kernel duration; --serial-views "
                                "times the kernel alone)"}
    kernels = {
        "raster_fused": raster_entry,
        "grad_adam_batch": {"ms": round(update_ms, 4), "bound": "hbm", "algorithmic_bytes": int(by),
                            "achieved_GBs": round(by / (update_ms * 1e-3) / 1e9, 1),
                            "frac": round(by / (update_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "note": "per optimiser step"},
    }
    from differentiable_rasterization_amd.profiling import read_stored_traffic
    stored = lambda k: read_stored_traffic(TRAFFIC_SUMMARY[k], k) if args.workload == "1m" else None
    if update_ms > raster_ms or vstreams is not None:
        d = kernels["grad_adam_batch"]
        roof = {"kernel": "k_grad_adam_batch", "bound": "hbm", "achieved": d["achieved_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": d["frac"], "traffic": stored("k_grad_adam_batch"),
                "algorithmic_bytes": d["algorithmic_bytes"], "launch_ms": d["ms"]}
    else:
        d = kernels["raster_fused"]
        roof = alu_roofline("k_raster_fused_l1", "raster_fused", d, walk_view, isect_view,
                            stored("k_raster_fused_l1"))
    out = {
        "metric": METRIC_OF[args.workload], "value": round(isect_total / wall, 1),
        "unit": "Gaussian-pixel intersections/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "ms_per_view": round(wall * 1e3 / (args.steps * bs), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": desc, "gaussians": n, "sh_degree": scene.sh_degree, "image": [W, H],
                   "views": nviews, "batch": bs, "binning_launch": "HIP graph per view" if use_graph[0] else "eager",
                   "binning_launch_trials_ms_per_step": launch_trials,
                   "views_on": "one stream each" if vstreams is not None else "one stream",
                   "step": f"one optimiser step over {bs} views: per view binning + fwd + L1 + bwd; one pass of "
                           "gradient mean, Adam (batch hyper-parameters) and the next batch's projections"},
        "roofline": roof,
        "intersections_per_view": round(isect_view, 1),
        "tile_entries_per_view": round(k_mean, 1),
        "kernels": kernels,
        "device": torch.cuda.get_device_name(0),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "20m":
        return main_partitioned(args)
    if args.batch != 1:
        if not 2 <= args.batch <= 4:
            print("--batch takes 1 to 4 views", file=sys.stderr)
            sys.exit(2)
        return main_batch(args)
    import torch
    from differentiable_rasterization_amd import binding as B
    from differentiable_rasterization_amd import pipeline as PL
    from differentiable_rasterization_amd.profiling import read_stored_traffic

    dev = "cuda"
    scene, desc = make_scene(args.workload)
    # both oracle legs run before anything touches the GPU: the parallel one forks, the
    # single-core one pins this thread to one core
    cpu_par = cpu_one = None
    if not args.no_cpu_baseline:
        cpu_par = cpu_baseline_parallel(scene, min(args.cpu_rows, scene.cameras[0].height))
        cpu_one = cpu_baseline(scene, min(args.cpu_rows, scene.cameras[0].height))
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
    # the binning of each view as a HIP graph (about thirty launches replayed as one); each
    # replay writes (K, required capacity or 0) to its view's counts and adds them to acc
    view_counts = torch.zeros(nviews, 2, dtype=torch.int64, device=dev)
    acc = torch.zeros(2, dtype=torch.int64, device=dev)
    graphs = None
    if args.binning_launch != "eager":
        B.gs_project(params.gaussians(), cams[0], st.raster, st.proj.abi())
        graphs = [PL.BinSortGraph(st.bins, st.proj, cams[v], st.raster, view_counts[v], acc) for v in range(nviews)]
    use_graph = [graphs is not None]

    if args.loss == "l1_dssim":
        args.separate_raster = True   # the structural term needs the whole image before the backward
    if args.unfused:
        names = ["project", "bin_sort", "raster_fwd", "loss", "raster_bwd", "grad_aggregate", "project_bwd", "adam"]
    elif args.separate_raster:   # the projection of each step runs in the previous step's last pass
        names = ["bin_sort", "raster_fwd", "loss", "raster_bwd", "grad_adam_project"]
    else:   # and forward, loss and backward rasterization run as one kernel
        names = ["bin_sort", "raster_fused", "grad_adam_project"]
    g = params.gaussians()

    # the calls timed inside the timed steps: the two kernels that can dominate the step
    timed_calls = [names.index(nm) for nm in ("raster_fused", "raster_bwd", "grad_adam", "grad_adam_project")
                   if nm in names]
    timed_marks = set(timed_calls) | {k + 1 for k in timed_calls}

    def one_step(i, ev=None, counts=None, every_call=False):
        """ev: HIP events, recorded around the dominant kernel's call only (each record costs
        the stream a few microseconds), or around every call if every_call."""
        c, t, nc = cams[i % nviews], targets[i % nviews], cams[(i + 1) % nviews]
        if ev is None:
            rec = lambda k: None
        elif every_call:
            rec = lambda k: ev[k].record()
        else:
            rec = lambda k: ev[k].record() if k in timed_marks else None
        f = st.frame
        k = 0
        rec(k)
        if args.unfused:
            B.gs_project(g, c, st.raster, st.proj.abi())
            k += 1
            rec(k)
        if use_graph[0]:   # no host wait; acc collects the counts
            graphs[i % nviews].replay()
        elif counts is None:
            st.bins.sort(st.proj, c, st.raster)
        else:   # no host wait inside the step; the counts are checked after the timed steps
            st.bins.sort_async(st.proj, c, st.raster, counts)
        rec(k + 1)
        if not args.unfused and not args.separate_raster:   # forward + L1 + backward in one kernel
            st.fused_l1(c, t)
            rec(k + 2)
            st.aggregate_adam_project(c, nc)
            rec(k + 3)
            return
        B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), c, st.raster, f.color, f.t_final, f.n_trav, f.n_trav_sum)
        rec(k + 2)
        if args.loss == "l1_dssim":
            st.loss_dssim(t, 0.2)
        else:
            B.gs_loss_l1(f.color, t, f.n_px, f.loss, f.dL_dcolor, f.loss_ws)
        rec(k + 3)
        B.gs_raster_bwd_partials(g, st.bins.abi(), c, st.raster, f.color, f.t_final, f.n_trav, f.dL_dcolor, None)
        rec(k + 4)
        if args.unfused:
            B.gs_grad_aggregate(g, st.proj.abi(), st.bins.abi(), c, st.raster, st.grads2d, None)
            rec(k + 5)
            st.backward_project(c)
            rec(k + 6)
            st.adam()
            rec(k + 7)
        else:   # per-Gaussian sum, projection backward, Adam and the next view's projection in one pass
            st.aggregate_adam_project(c, nc)
            rec(k + 5)

    def project_for(i):
        """The records step i starts from (the fused pass projects for the step after it)."""
        if not args.unfused:
            B.gs_project(g, cams[i % nviews], st.raster, st.proj.abi())

    if args.copy_calibration_mib > 0:
        # a copy-like kernel of known size (reads and writes M MiB) for counter normalisation
        src = torch.ones(args.copy_calibration_mib << 18, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    project_for(0)
    quiet_gc()
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    step0 = args.warmup
    launch_trials = None
    if args.binning_launch == "auto":
        launch_trials = choose_binning_launch(one_step, use_graph, step0, max(2 * nviews, 4), 1)
        step0 += launch_trials.pop("steps")
    new_events = lambda: [[TimingEvent() for _ in range(len(names) + 1)]
                          for _ in range(args.steps)]
    events = new_events()
    st.frame.n_trav_sum.zero_()
    counts = torch.zeros(args.steps, 2, dtype=torch.int64, device=dev)
    acc.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(step0 + i, events[i], counts[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    if use_graph[0]:
        k_sum, need = (int(x) for x in acc.cpu())
        if need != 0:
            raise RuntimeError("intersection lists overflowed during the timed steps")
        k_isect = [k_sum / args.steps]
    else:
        cnt = counts.cpu()
        if int(cnt[:, 1].max()) != 0:
            raise RuntimeError(f"intersection lists overflowed during the timed steps (need {int(cnt[:, 1].max())})")
        k_isect = [int(k) for k in cnt[:, 0]]
    # quadrant records of the last sort (the list header: entries, then quadrant records)
    q_last = int(st.bins.raster[:16].view(torch.int64)[1].item())
    isect_total = int(st.frame.n_trav_sum.item())
    timed_ms = {names[k]: sum(events[s][k].elapsed_time(events[s][k + 1]) for s in range(args.steps)) / args.steps
                for k in timed_calls}
    per_kernel, step_ms = dict(timed_ms), None
    if not args.no_breakdown:
        # untimed: the same steps again with an event around every call
        project_for(step0)
        ev2 = new_events()
        for i in range(args.steps):
            one_step(step0 + i, ev2[i], counts[i], every_call=True)
        torch.cuda.synchronize()
        per_kernel = {names[j]: sum(ev2[s][j].elapsed_time(ev2[s][j + 1]) for s in range(args.steps)) / args.steps
                      for j in range(len(names))}
        per_kernel.update(timed_ms)
        step_ms = sorted(ev2[s][0].elapsed_time(ev2[s][-1]) for s in range(args.steps))
    # the raster walks, counted on the device by the fused kernel's counting instance: one
    # untimed call on each view's lists (projected and sorted from the current parameters),
    # weighted by how often each view ran in the timed steps
    def count_view(v):
        def run(wc):
            B.gs_project(g, cams[v], st.raster, st.proj.abi())
            st.bins.sort(st.proj, cams[v], st.raster)
            st.fused_l1(cams[v], targets[v], walk_counts=wc)
        return run
    walks = count_walks([count_view(v) for v in range(nviews)])
    wts = [sum(1 for i in range(args.steps) if (step0 + i) % nviews == v) for v in range(nviews)]
    walk_step = [sum(w * wk[j] for w, wk in zip(wts, walks)) / args.steps for j in range(3)]
    # ByteSplat Eq. 7-9 for the last step's tile lists: how many tiles a design that keeps a
    # tile's records on chip could hold (64 KiB of LDS per tile, 256 pixels x 32 B of pixel
    # state, 48-B records); the fused kernel streams records and runs every tile
    lds_budget, fixed_bytes, rec_bytes = 64 * 1024, 256 * 32, 48
    budget = B.gs_tile_budget(lds_budget, fixed_bytes, rec_bytes)
    totals = torch.zeros(2, dtype=torch.int64, device=dev)
    B.gs_tile_budget_report(st.bins.abi(), cams[(args.warmup + args.steps - 1) % nviews], budget, None, None, totals)
    tiles_over, excess = (int(x) for x in totals.cpu())
    tile_budget = {"B": budget, "lds_budget_bytes": lds_budget, "fixed_bytes": fixed_bytes, "bytes_per_gaussian": rec_bytes,
                   "tiles": st.bins.tiles, "tiles_over_budget": tiles_over,
                   "frac_tiles_within": round(1.0 - tiles_over / st.bins.tiles, 4), "sum_excess": excess}
    # the realized skew of the last step's tile lists: longest over mean list, and the share of
    # the entries in the longest 1 % of tiles; for the clustered 10M scene also the share of
    # the means inside the dense central sub-cube (10 % of the 20 m cube's volume)
    lens = (st.bins.tile_ranges[1:] - st.bins.tile_ranges[:-1]).to(torch.float64)
    top = max(1, lens.numel() // 100)
    skew = {"tile_list_max_over_mean": round(float(lens.max()) / max(float(lens.mean()), 1e-30), 2),
            "top1pct_tiles_share_of_entries": round(float(lens.topk(top).values.sum()) / max(float(lens.sum()), 1.0), 4)}
    if args.workload == "10m":
        sub_half = 10.0 * 0.1 ** (1.0 / 3.0)
        skew["means_in_dense_subcube"] = round(float((scene.means.abs() <= sub_half).all(dim=0).double().mean()), 4)
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
        elif nm in ALU_KERNELS:
            entry.update(alu_entry(nm, ms, walk_step, isect_step))
        kernels[nm] = entry
    def roofline(nm):
        d = kernels[nm]
        kern = KERNEL_OF[nm]
        traffic = read_stored_traffic(TRAFFIC_SUMMARY[kern], kern) if args.workload == "1m" else None
        if d["bound"] == "alu":
            return alu_roofline(kern, nm, d, walk_step, isect_step, traffic)
        return {"kernel": kern, "bound": "hbm", "achieved": d["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac"], "traffic": traffic, "algorithmic_bytes": d["algorithmic_bytes"],
                "launch_ms": d["ms"]}

    # the dominant kernel: the longer of the two timed in the timed steps
    ranked = sorted(timed_ms, key=timed_ms.get, reverse=True)
    roof = roofline(ranked[0])
    roof_next = roofline(ranked[1]) if len(ranked) > 1 else None
    out = {
        "metric": METRIC_OF[args.workload], "value": round(isect_total / wall, 1),
        "unit": "Gaussian-pixel intersections/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": desc, "gaussians": n, "sh_degree": scene.sh_degree, "image": [W, H],
                   "views": nviews,
                   "loss": "L1" if args.loss == "l1" else "(1 - 0.2) L1 + 0.2 (1 - SSIM) / 2",
                   "step": "one view: projection + fwd + L1 + bwd + Adam" + (
                       "" if args.unfused else " (each view's projection fused into the previous step's Adam pass"
                       + ("" if args.separate_raster else "; fwd + L1 + bwd in one kernel") + ")"),
                   "binning_launch": "HIP graph per view" if use_graph[0] else "eager",
                   "binning_launch_trials_ms_per_step": launch_trials},
        "roofline": roof,
        "roofline_next": roof_next,
        # from the untimed pass with an event around every call
        "step_stream_ms": {"median": round(step_ms[len(step_ms) // 2], 4),
                           "p90": round(step_ms[min(len(step_ms) - 1, int(0.9 * len(step_ms)))], 4)}
        if step_ms else None,
        "intersections_per_step": round(isect_step, 1),
        "tile_entries_per_step": round(kmean, 1),
        "quadrant_records_last_step": q_last,
        "visible_gaussians": n_vis,
        "tile_budget": tile_budget,
        "skew": skew,
        # Gaussian-pixel intersections over the two raster kernels' time (forward compositing
        # and the per-pixel backward with its per-quadrant sums)
        "raster_isect_per_s": round(isect_step / ((per_kernel["raster_fwd"] + per_kernel["raster_bwd"]) * 1e-3), 1)
        if "raster_fwd" in per_kernel else round(isect_step / (per_kernel["raster_fused"] * 1e-3), 1),
        "kernels_note": "raster_fused (or raster_bwd) and grad_adam(_project) from events in the timed steps; the others "
                        "from an untimed "
                        "pass of the same steps with an event around every call",
        "kernels": kernels,
        "device": torch.cuda.get_device_name(0),
        "device_info": device_info(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_one
        out["cpu_baseline_parallel"] = cpu_par
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
