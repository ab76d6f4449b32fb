"""Device buffers and the call sequence of one training step.

Allocation (torch, on the GPU) and the order of the C-ABI calls only; every step
of the computation runs in libgsmi's kernels:

    gs_project -> gs_bin_sort -> gs_raster_fwd -> gs_loss_l1 -> gs_raster_bwd -> gs_adam_step

of one training step over depth slabs rendered separately and over-composited
(PartitionedStep), and of one training step over a batch of views (BatchTrainStep).

Parameters, gradients and the two Adam moments each live in one [planes][LD]
float32 buffer (structure of arrays, LD = N rounded up to 64), so every kernel
streams coalesced planes whose 64-Gaussian segments cover whole cache lines, and
Adam runs as one launch over six parameter groups.
"""
from __future__ import annotations

import math

import torch

from . import binding as B

# reading: the pages give Adam's eps and betas but no learning rates; these are
# per-group defaults of the common 3DGS recipe
DEFAULT_LR = dict(means=1.6e-4, log_scales=5e-3, quats=1e-3, opacity_logits=5e-2, sh_dc=2.5e-3, sh_rest=1.25e-4)


class GaussianParams:
    """Learnable parameters plus gradients and Adam moments, structure of arrays.

    Each set is stored as [planes][ld] with ld = n rounded up to 64 (a plane stride whose
    64-Gaussian segments start on 256-byte boundaries; the per-Gaussian kernels run up to
    twice as long on planes that straddle cache lines).  data, grad, m and v are the
    [planes][n] views; the padding stays zero (Adam leaves zero entries at zero)."""

    LD_ALIGN = 64

    def __init__(self, n: int, sh_degree: int, device="cuda"):
        self.n, self.sh_degree = n, sh_degree
        self.k_sh = (sh_degree + 1) ** 2
        self.planes = 11 + 3 * self.k_sh
        self.ld = -(-n // self.LD_ALIGN) * self.LD_ALIGN
        z = lambda: torch.zeros(self.planes, self.ld, dtype=torch.float32, device=device)
        self.store = dict(data=z(), grad=z(), m=z(), v=z())
        self.data, self.grad, self.m, self.v = (self.store[k][:, :n] for k in ("data", "grad", "m", "v"))
        self.step_count = 0

    _SLICES = (("means", 0, 3), ("log_scales", 3, 6), ("quats", 6, 10), ("opacity_logits", 10, 11))

    def view(self, buf, name):
        for nm, a, b in self._SLICES:
            if nm == name:
                return buf[a:b] if b - a > 1 else buf[a]
        if name == "sh":
            return buf[11:]
        raise KeyError(name)

    @classmethod
    def from_scene(cls, scene, device="cuda"):
        p = cls(scene.n, scene.sh_degree, device)
        for name in ("means", "log_scales", "quats", "opacity_logits", "sh"):
            p.view(p.data, name).copy_(getattr(scene, name).to(device))
        return p

    def gaussians(self) -> B.Gaussians:
        v = lambda nm: self.view(self.data, nm)
        return B.gaussians(v("means"), v("log_scales"), v("quats"), v("opacity_logits"), v("sh"))

    def param_grads(self) -> B.ParamGrads:
        v = lambda nm: self.view(self.grad, nm)
        return B.param_grads(v("means"), v("log_scales"), v("quats"), v("opacity_logits"), v("sh"))

    def moments(self):
        """(m, v) as ABI parameter sets."""
        def ps(buf):
            v = lambda nm: self.view(buf, nm)
            return B.param_grads(v("means"), v("log_scales"), v("quats"), v("opacity_logits"), v("sh"))
        return ps(self.m), ps(self.v)

    def adam_groups(self, lr=DEFAULT_LR):
        """Six flat groups over the padded rows (the padding has zero gradients and moments,
        so Adam leaves it at zero)."""
        bounds = [("means", 0, 3), ("log_scales", 3, 6), ("quats", 6, 10), ("opacity_logits", 10, 11),
                  ("sh_dc", 11, 14), ("sh_rest", 14, self.planes)]
        st = self.store
        out = []
        for name, a, b in bounds:
            if b <= a:
                continue
            out.append((st["data"][a:b], st["grad"][a:b], st["m"][a:b], st["v"][a:b], lr[name]))
        return out


class Projection:
    """Projected records of n Gaussians: depth keys, radii and the raster records, and with
    plain=True also the plain record fields as planes (means2d [2][n], conic_opacity [4][n],
    color [3][n]), which the training step itself never reads."""

    def __init__(self, n, device="cuda", plain=False):
        n = max(n, 1)   # the raster entry points take the record pointers even for an empty scene
        z = lambda *shape: torch.zeros(*shape, dtype=torch.float32, device=device)
        self.means2d = z(2, n) if plain else None
        self.conic_opacity = z(4, n) if plain else None
        self.color = z(3, n) if plain else None
        self.depth = z(n)
        self.radii = torch.zeros(n, 2, dtype=torch.int32, device=device)
        self.rec = z(n, 12)   # raster record

    def abi(self) -> B.Projected:
        return B.projected(self.means2d, self.conic_opacity, self.color, self.depth, self.radii, self.rec)


class Binning:
    """Intersection lists and the sort workspace; grows on demand."""

    def __init__(self, n, width, height, capacity=0, device="cuda", with_keys=False, with_touched=False):
        self.n, self.width, self.height, self.device = n, width, height, device
        self.tiles = ((width + 15) // 16) * ((height + 15) // 16)
        self.tile_ranges = torch.zeros(self.tiles + 1, dtype=torch.int32, device=device)
        self.with_keys, self.with_touched = with_keys, with_touched
        self.tiles_touched = torch.zeros(n, dtype=torch.int32, device=device) if with_touched else None
        self.n_isect = 0
        self._alloc(max(capacity, 1))

    def _alloc(self, capacity):
        self.capacity = int(capacity)
        self.ids = torch.zeros(self.capacity, dtype=torch.int32, device=self.device)
        self.keys = torch.zeros(self.capacity, dtype=torch.int64, device=self.device) if self.with_keys else None
        ws = B.gs_bin_sort_workspace_bytes(self.n, self.capacity, self.width, self.height)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.device)
        rb = B.gs_bins_raster_bytes(self.n, self.capacity, self.width, self.height)
        self.raster = torch.empty(max(rb, 256), dtype=torch.uint8, device=self.device)

    def abi(self) -> B.Bins:
        return B.bins(self.ids, self.tile_ranges, self.raster, self.keys, self.tiles_touched)

    def sort(self, proj: Projection, cam: B.Camera, params: B.RasterParams, stream=None) -> int:
        try:
            k = B.gs_bin_sort(proj.abi(), self.n, cam, params, self.abi(), self.workspace, stream)
        except B.GsCapacityError as e:
            self._alloc(int(math.ceil(e.required * 1.25)) + 1024)
            k = B.gs_bin_sort(proj.abi(), self.n, cam, params, self.abi(), self.workspace, stream)
        self.n_isect = k
        return k

    def sort_async(self, proj: Projection, cam: B.Camera, params: B.RasterParams, counts=None, stream=None):
        """Queues the sort without a host wait; counts (device int64[2]) receives (K,
        required capacity or 0).  The caller checks it and repeats the step after growing."""
        B.gs_bin_sort_async(proj.abi(), self.n, cam, params, self.abi(), counts, self.workspace, stream)


class BinSortGraph:
    """gs_bin_sort_async for one camera, captured once as a HIP graph and replayed.

    The sort is about thirty small kernel launches; on a slow host their launch cost
    exceeds their GPU time and the step waits for the host.  A replay is one launch.
    The graph holds the buffers' addresses and the camera: it stays valid while bins,
    proj and counts keep their storage (Binning._alloc replaces it).  Every kernel of
    the sort clears what it needs with its own stores (no memset nodes).  With acc
    (device int64[2]), each replay also adds counts to it (entries, required capacity):
    acc[1] != 0 after a run means some sort overflowed."""

    def __init__(self, bins: Binning, proj: Projection, cam: B.Camera, params: B.RasterParams, counts,
                 acc=None):
        self.bins, self.counts = bins, counts
        self._storage = (bins.ids.data_ptr(), bins.workspace.data_ptr(), bins.raster.data_ptr())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # one eager run first, off the capture
            bins.sort_async(proj, cam, params, counts)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            bins.sort_async(proj, cam, params, counts)
            if acc is not None:
                acc.add_(counts)

    def replay(self):
        b = self.bins
        if (b.ids.data_ptr(), b.workspace.data_ptr(), b.raster.data_ptr()) != self._storage:
            raise RuntimeError("the binning buffers were reallocated after the graph was captured")
        self.graph.replay()


class Frame:
    """Per-image buffers: render, transmittance, traversal counts, loss gradient."""

    def __init__(self, width, height, device="cuda"):
        self.width, self.height = width, height
        self.n_px = width * height
        self.color = torch.zeros(height, width, 3, dtype=torch.float32, device=device)
        self.t_final = torch.zeros(height, width, dtype=torch.float32, device=device)
        self.n_trav = torch.zeros(height, width, dtype=torch.int32, device=device)
        self.dL_dcolor = torch.zeros(height, width, 3, dtype=torch.float32, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        # running sum of N_p (Gaussian-pixel evaluations) over forward passes; cleared by the caller
        self.n_trav_sum = torch.zeros(1, dtype=torch.int64, device=device)
        self.loss_ws = torch.empty(max(B.gs_loss_workspace_bytes(self.n_px), 8), dtype=torch.uint8, device=device)
        self.ssim = torch.zeros(1, dtype=torch.float32, device=device)
        self.ssim_ws = None   # allocated on the first D-SSIM loss
        # per-wave partial sums of the fused forward + L1 + backward
        self.fused_ws = torch.empty(max(B.gs_raster_fused_l1_workspace_bytes(width, height), 16),
                                    dtype=torch.uint8, device=device)


class TrainStep:
    """One-view training step on one GPU: forward, L1 loss, backward, Adam."""

    def __init__(self, params: GaussianParams, width, height, device="cuda", raster=None, lr=DEFAULT_LR,
                 capacity=0, plain=False):
        self.params = params
        self.raster = raster if raster is not None else B.make_params(params.sh_degree)
        self.proj = Projection(params.n, device, plain)
        self.bins = Binning(params.n, width, height, capacity=capacity, device=device)
        self.frame = Frame(width, height, device)
        self.grads2d = torch.zeros(9, max(params.n, 1), dtype=torch.float32, device=device)
        self.lr = lr

    def forward(self, cam: B.Camera, stream=None):
        B.gs_project(self.params.gaussians(), cam, self.raster, self.proj.abi(), stream)
        self.forward_projected(cam, stream)

    def forward_projected(self, cam: B.Camera, stream=None):
        """Binning and forward rasterization of the records already in self.proj (written by
        gs_project or by aggregate_adam_project for this camera)."""
        self.bins.sort(self.proj, cam, self.raster, stream)
        f = self.frame
        B.gs_raster_fwd(self.proj.abi(), self.bins.abi(), cam, self.raster, f.color, f.t_final, f.n_trav,
                        f.n_trav_sum, stream)

    def loss(self, target, stream=None):
        f = self.frame
        B.gs_loss_l1(f.color, target, f.n_px, f.loss, f.dL_dcolor, f.loss_ws, stream)

    def loss_dssim(self, target, lam=0.2, stream=None):
        """(1 - lam) L1 + lam (1 - SSIM) / 2 into frame.loss (and frame.ssim), its gradient into
        frame.dL_dcolor; follow with backward_partials and the end-of-step pass."""
        f = self.frame
        if f.ssim_ws is None:
            f.ssim_ws = torch.empty(B.gs_loss_l1_dssim_workspace_bytes(f.width, f.height), dtype=torch.uint8,
                                    device=f.color.device)
        B.gs_loss_l1_dssim(f.color, target, f.width, f.height, lam, f.loss, f.ssim, f.dL_dcolor, f.ssim_ws, stream)

    def backward_raster(self, cam: B.Camera, dL_dcolor=None, dL_dt=None, stream=None):
        f = self.frame
        B.gs_raster_bwd(self.params.gaussians(), self.proj.abi(), self.bins.abi(), cam, self.raster, f.color,
                        f.t_final, f.n_trav, f.dL_dcolor if dL_dcolor is None else dL_dcolor, dL_dt, self.grads2d, None,
                        stream)

    def backward_project(self, cam: B.Camera, stream=None):
        B.gs_project_bwd(self.params.gaussians(), cam, self.raster, self.grads2d, self.params.param_grads(), stream)

    def backward(self, cam: B.Camera, dL_dcolor=None, dL_dt=None, stream=None, grads3d=True):
        self.backward_raster(cam, dL_dcolor, dL_dt, stream)
        if grads3d:
            self.backward_project(cam, stream)

    def adam(self, stream=None):
        self.params.step_count += 1
        B.gs_adam_step(self.params.adam_groups(self.lr), self.params.step_count, 0.9, 0.999, 1e-15, stream)

    def aggregate_adam(self, cam: B.Camera, grads2d=None, stream=None):
        """Per-Gaussian gradient sum, projection backward and Adam in one pass (after
        backward_partials); the 3D gradients are not stored."""
        self.params.step_count += 1
        m, v = self.params.moments()
        B.gs_grad_aggregate_adam(self.params.gaussians(), self.proj.abi(), self.bins.abi(), cam, self.raster, grads2d, m, v,
                                 B.AdamLrs(**self.lr), self.params.step_count, 0.9, 0.999, 1e-15, stream)

    def aggregate_adam_project(self, cam: B.Camera, next_cam: B.Camera, grads2d=None, stream=None):
        """aggregate_adam, then the projection of the updated Gaussians for next_cam into
        self.proj in the same pass (the next step then starts at the binning)."""
        self.params.step_count += 1
        m, v = self.params.moments()
        pa = self.proj.abi()
        B.gs_grad_aggregate_adam_project(self.params.gaussians(), pa, self.bins.abi(), cam, self.raster, grads2d, m,
                                         v, B.AdamLrs(**self.lr), self.params.step_count, 0.9, 0.999, 1e-15,
                                         next_cam, pa, stream)

    def fused_l1(self, cam: B.Camera, target, stream=None, walk_counts=None):
        """Forward rasterization, L1 loss and the per-record backward in one kernel (from the
        current bins); equal to forward rasterization, loss and backward_partials.  With
        walk_counts (device int64[3]) the counting instance runs and adds the records walked
        forward and backward and the accepted pairs."""
        f = self.frame
        B.gs_raster_fused_l1(self.params.gaussians(), self.bins.abi(), cam, self.raster, target, f.color, f.t_final,
                             f.n_trav, f.loss, f.n_trav_sum, f.fused_ws, stream, walk_counts=walk_counts)

    def backward_partials(self, cam: B.Camera, dL_dcolor=None, dL_dt=None, stream=None):
        f = self.frame
        B.gs_raster_bwd_partials(self.params.gaussians(), self.bins.abi(), cam, self.raster, f.color, f.t_final,
                                 f.n_trav, f.dL_dcolor if dL_dcolor is None else dL_dcolor, dL_dt, stream)

    def step(self, cam: B.Camera, target, stream=None):
        self.forward(cam, stream)
        self.loss(target, stream)
        self.backward(cam, stream=stream)
        self.adam(stream)


class ViewStreams:
    """One stream per view of a batch.  fork() makes each stream wait for everything queued
    on the caller's stream so far; join() makes the caller's stream wait for all of them.
    The views' binning and rasterization are independent (each has its own bins, frame and
    gradient slots; the parameters are only read), and a binning is a chain of small
    kernels that leaves most of the GPU idle, so the views' chains run side by side.  The
    streams keep the default priority."""

    def __init__(self, views):
        self.streams = [torch.cuda.Stream() for _ in range(views)]

    def fork(self):
        main = torch.cuda.current_stream()
        for s in self.streams:
            s.wait_stream(main)

    def join(self):
        main = torch.cuda.current_stream()
        for s in self.streams:
            main.wait_stream(s)


class BatchTrainStep:
    """One optimiser step over a batch of views (ROCm blog, "Batching and Hyperparameter
    Scaling": several camera views per step, learning rates times sqrt(BS), eps / sqrt(BS),
    betas 1 - BS (1 - beta)).  The Gaussians are projected for all views of the batch in one
    pass (gs_project_batch); each view is binned and runs the fused forward + L1 + backward
    (the loss of the batch is the mean of the views' L1 losses); one pass per Gaussian then
    adds the views' gradients, applies Adam and projects the updated Gaussians for the next
    batch's views (gs_grad_aggregate_adam_batch)."""

    MAX_VIEWS = 4

    def __init__(self, params: GaussianParams, width, height, views, device="cuda", raster=None, lr=DEFAULT_LR,
                 capacity=0):
        if not 1 <= views <= self.MAX_VIEWS:
            raise ValueError(f"views must lie in [1, {self.MAX_VIEWS}]")
        self.params, self.views = params, views
        self.raster = raster if raster is not None else B.make_params(params.sh_degree)
        self.proj = [Projection(params.n, device) for _ in range(views)]
        self.bins = [Binning(params.n, width, height, capacity=capacity, device=device) for _ in range(views)]
        self.frame = [Frame(width, height, device) for _ in range(views)]
        self.lrs, self.beta1, self.beta2, self.eps = B.gs_adam_batch_hparams(views, B.AdamLrs(**lr))

    def project(self, cams, stream=None):
        B.gs_project_batch(self.params.gaussians(), cams, self.raster, [p.abi() for p in self.proj], stream)

    def sort(self, k, cam: B.Camera, stream=None):
        self.bins[k].sort(self.proj[k], cam, self.raster, stream)

    def render(self, k, cam: B.Camera, target, stream=None):
        """View k: forward, L1 loss and the per-record backward in one kernel."""
        f = self.frame[k]
        B.gs_raster_fused_l1(self.params.gaussians(), self.bins[k].abi(), cam, self.raster, target, f.color,
                             f.t_final, f.n_trav, f.loss, f.n_trav_sum, f.fused_ws, stream)

    def update(self, cams, next_cams=None, stream=None):
        """The views' gradients (mean over the batch), Adam and, with next_cams, the next
        batch's projections into self.proj."""
        self.params.step_count += 1
        m, v = self.params.moments()
        nxt = [p.abi() for p in self.proj] if next_cams is not None else None
        B.gs_grad_aggregate_adam_batch(self.params.gaussians(), [b.abi() for b in self.bins], cams, self.raster,
                                       1.0 / self.views, m, v, self.lrs, self.params.step_count, self.beta1,
                                       self.beta2, self.eps, next_cams, nxt, stream)

    def step(self, cams, targets, next_cams=None, view_streams: ViewStreams | None = None):
        """The batch's projections must be in self.proj (project(), or the previous step's
        update with next_cams).  With view_streams, each view is binned and rasterized on
        its own stream (on the current stream otherwise); the update runs on the current
        stream after all of them."""
        if view_streams is not None:
            view_streams.fork()
        for k in range(self.views):
            if view_streams is not None:
                with torch.cuda.stream(view_streams.streams[k]):
                    self.sort(k, cams[k])
                    self.render(k, cams[k], targets[k])
            else:
                self.sort(k, cams[k])
                self.render(k, cams[k], targets[k])
        if view_streams is not None:
            view_streams.join()
        self.update(cams, next_cams)


class PartitionedStep:
    """One view's training step over Gaussians split into camera-space depth slabs.

    Forward: each slab projects, bins and composites its own Gaussians into a partial
    image (C_k, T_k); the partials are over-composited in depth order (Splaxel sections
    3.4 and 4.2: convex partitions in depth order reproduce the global blending order;
    section 4.3: partitions behind a saturated pixel are skipped).  Loss: L1 on the
    composite.  Backward: the composite backward gives each slab (dL/dC_k, dL/dT_k); each
    slab's backward rasterization and per-Gaussian sum give its screen-space gradients,
    which are compacted to the records of non-zero Gaussians (ByteSplat section 6.1) and
    decoded into the owner's gradient planes (section 6.2).  On one GPU a slab's renderer
    and owner are the same; the exchange between them is left out.  The owner then runs
    the projection backward and Adam for its Gaussians in one pass (gs_project_bwd_adam),
    which with next_cam also projects the updated slab for the next step's camera, so that
    the next step (projected=True) starts at the binning.

    slabs: one GaussianParams per slab (disjoint Gaussians); windows: the slabs' depth
    windows [lo, hi) of the projection (Gaussians outside are culled)."""

    def __init__(self, slabs, windows, width, height, device="cuda", t_min=1e-4, lr=DEFAULT_LR, capacity=0):
        self.width, self.height, self.t_min = width, height, t_min
        self.n_px = width * height
        self.parts = []
        for params, (lo, hi) in zip(slabs, windows):
            rp = B.make_params(params.sh_degree, t_min=t_min, depth_lo=lo, depth_hi=hi)
            self.parts.append(TrainStep(params, width, height, device, raster=rp, lr=lr, capacity=capacity))
        z = lambda *shape: torch.zeros(*shape, dtype=torch.float32, device=device)
        self.color, self.t_final = z(height, width, 3), z(height, width)
        self.loss_value, self.dL_dcolor = z(1), z(height, width, 3)
        self.loss_ws = torch.empty(max(B.gs_loss_workspace_bytes(self.n_px), 8), dtype=torch.uint8, device=device)
        self.ssim = torch.zeros(1, dtype=torch.float32, device=device)
        self.ssim_ws = None   # allocated on the first D-SSIM loss
        self.dcs = [z(height, width, 3) for _ in self.parts]
        self.dts = [z(height, width) for _ in self.parts]
        self.records, self.bitmaps, self.compact_ws, self.owner_g2, self.r = [], [], [], [], []
        for st in self.parts:
            n = max(st.params.n, 1)
            self.records.append(torch.zeros(n, 10, dtype=torch.int32, device=device))
            self.bitmaps.append(torch.zeros((n + 31) // 32, dtype=torch.int32, device=device))
            self.compact_ws.append(torch.empty(max(B.gs_compact_workspace_bytes(n), 256), dtype=torch.uint8,
                                               device=device))
            self.owner_g2.append(z(9, n))
            self.r.append(0)
        self.streams = None   # ViewStreams of the overlapped schedule, made on first use
        # (K, required capacity or 0) of each slab's binning in the overlapped schedule
        self.counts = torch.zeros(len(self.parts), 2, dtype=torch.int64, device=device)

    # -- forward
    def render_part(self, k, cam: B.Camera, stream=None):
        self.parts[k].forward(cam, stream)

    def composite(self, stream=None):
        B.gs_composite_over([st.frame.color for st in self.parts], [st.frame.t_final for st in self.parts],
                            self.n_px, self.t_min, self.color, self.t_final, stream)

    def forward(self, cam: B.Camera, stream=None, projected=False):
        """projected: each slab's projection buffers already hold its projection for cam
        (written by the previous step's update with next_cam = cam)."""
        for k, st in enumerate(self.parts):
            if projected:
                st.forward_projected(cam, stream)
            else:
                self.render_part(k, cam, stream)
        self.composite(stream)

    def loss(self, target, stream=None):
        B.gs_loss_l1(self.color, target, self.n_px, self.loss_value, self.dL_dcolor, self.loss_ws, stream)

    # -- backward
    def composite_backward(self, stream=None):
        B.gs_composite_over_bwd([st.frame.color for st in self.parts], [st.frame.t_final for st in self.parts],
                                self.n_px, self.t_min, self.dL_dcolor, None, self.dcs, self.dts, stream)

    def backward_part(self, k, cam: B.Camera, stream=None):
        """The slab's backward rasterization and per-Gaussian sum into its grads2d."""
        st = self.parts[k]
        st.backward_partials(cam, dL_dcolor=self.dcs[k], dL_dt=self.dts[k], stream=stream)
        B.gs_grad_aggregate(st.params.gaussians(), st.proj.abi(), st.bins.abi(), cam, st.raster, st.grads2d, None,
                            stream)

    def compact_part(self, k, stream=None) -> int:
        """Non-zero records of the slab's gradients (reads the count back to the host)."""
        st = self.parts[k]
        self.r[k] = B.gs_compact_grads(st.grads2d, st.params.n, 0, self.records[k], self.bitmaps[k],
                                       self.compact_ws[k], stream)
        return self.r[k]

    def decode_part(self, k, stream=None):
        """The owner's side: its gradient planes rebuilt from the slab's records."""
        n = self.parts[k].params.n
        self.owner_g2[k].zero_()
        B.gs_decode_grads([(self.records[k], self.r[k], 0, None, n)], self.owner_g2[k], n, None, stream)

    def update_part(self, k, cam: B.Camera, stream=None, next_cam: B.Camera = None):
        """The owner's projection backward from the decoded gradients and Adam in one pass;
        with next_cam, also the projection of the updated slab for next_cam into the slab's
        projection buffers.  The 3D gradients are not stored."""
        st = self.parts[k]
        st.params.step_count += 1
        m, v = st.params.moments()
        B.gs_project_bwd_adam(st.params.gaussians(), cam, st.raster, self.owner_g2[k], m, v, B.AdamLrs(**st.lr),
                              st.params.step_count, 0.9, 0.999, 1e-15, next_cam,
                              st.proj.abi() if next_cam is not None else None, stream)

    def update_part_separate(self, k, cam: B.Camera, stream=None):
        """update_part without next_cam as two calls: the projection backward into the
        slab's 3D gradients, then Adam (the same result, bit for bit)."""
        st = self.parts[k]
        B.gs_project_bwd(st.params.gaussians(), cam, st.raster, self.owner_g2[k], st.params.param_grads(), stream)
        st.adam(stream)

    def backward(self, cam: B.Camera, stream=None):
        self.composite_backward(stream)
        for k in range(len(self.parts)):
            self.backward_part(k, cam, stream)
            self.compact_part(k, stream)
            self.decode_part(k, stream)

    def step(self, cam: B.Camera, target, stream=None, next_cam: B.Camera = None, projected=False):
        self.forward(cam, stream, projected)
        self.loss(target, stream)
        self.backward(cam, stream)
        for k in range(len(self.parts)):
            self.update_part(k, cam, stream, next_cam)

    # -- the same step with the slabs side by side
    #
    # The slabs share nothing until the composite and nothing again after the composite
    # backward.  Each slab's projection and binning, and later its compaction, decoding and
    # update (projection backward and Adam: HBM-bound), run on a stream of its own; the
    # rasterizations (VALU-bound) run in slab order on one more stream, each after its
    # slab's binning, so that one slab's rasterization overlaps the other slabs' binning
    # and updates rather than the other rasterizations.  The binning does not wait for the
    # host (the lists must fit the buffers' capacity: self.counts[k] = (K, required
    # capacity or 0) tells after the step, check_capacity grows them); the whole backward
    # chain is queued before the first compaction reads its record count, so the later
    # slabs run while the host waits.  Every call is the serial step's, on the same data:
    # the results are the same bit for bit.

    def _slab_streams(self):
        if self.streams is None:
            self.streams = ViewStreams(len(self.parts) + 1)   # one per slab, then the raster stream
        return self.streams

    def forward_overlapped(self, cam: B.Camera, projected=False):
        vs = self._slab_streams()
        rs = vs.streams[-1]
        vs.fork()
        for k, st in enumerate(self.parts):
            with torch.cuda.stream(vs.streams[k]):
                if not projected:
                    B.gs_project(st.params.gaussians(), cam, st.raster, st.proj.abi())
                st.bins.sort_async(st.proj, cam, st.raster, self.counts[k])
        for k, st in enumerate(self.parts):
            rs.wait_stream(vs.streams[k])   # slab k's lists
            with torch.cuda.stream(rs):
                f = st.frame
                B.gs_raster_fwd(st.proj.abi(), st.bins.abi(), cam, st.raster, f.color, f.t_final, f.n_trav,
                                f.n_trav_sum)
        vs.join()
        self.composite()

    def backward_overlapped(self, cam: B.Camera, join=True, next_cam: B.Camera = None):
        """Composite backward, then each slab's backward rasterization and per-Gaussian sum
        on the raster stream, and its compaction, decoding and update on its own stream.
        join=False leaves the updates running: the next step_overlapped orders each slab's
        projection (with projected=True, its binning) after its own update (same stream)
        and everything else after those, so one slab's update overlaps the next step's
        binning of the others; call join() (or synchronize) before reading the parameters.
        next_cam: as in update_part."""
        vs = self._slab_streams()
        rs = vs.streams[-1]
        self.composite_backward()
        vs.fork()
        for k in range(len(self.parts)):
            with torch.cuda.stream(rs):
                self.backward_part(k, cam)
            vs.streams[k].wait_stream(rs)   # slab k's gradients
        for k in range(len(self.parts)):
            with torch.cuda.stream(vs.streams[k]):
                self.compact_part(k)   # waits for this slab's stream only
                self.decode_part(k)
                self.update_part(k, cam, next_cam=next_cam)
        if join:
            vs.join()

    def join(self):
        """Makes the current stream wait for the slabs' streams."""
        if self.streams is not None:
            self.streams.join()

    def step_overlapped(self, cam: B.Camera, target, join=True, next_cam: B.Camera = None, projected=False):
        self.forward_overlapped(cam, projected)
        self.loss(target)
        self.backward_overlapped(cam, join, next_cam)

    def check_capacity(self) -> bool:
        """After overlapped steps: True if every slab's lists fit; otherwise the short
        buffers are grown (the steps since the last check must be repeated)."""
        c = self.counts.cpu()
        ok = True
        for k, st in enumerate(self.parts):
            need = int(c[k, 1])
            if need:
                ok = False
                st.bins._alloc(int(math.ceil(need * 1.25)) + 1024)
            else:
                st.bins.n_isect = int(c[k, 0])
        return ok
