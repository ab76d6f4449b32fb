"""Seeded synthetic inputs for the Gaussian-splatting training step.

This module only draws random numbers and lays them out.  It holds none of
the rendering arithmetic (no projection, no spherical-harmonic evaluation, no
compositing); both the HIP library and the CPU oracle consume what it
returns, so nothing here may depend on either of them.

Layout (structure of arrays, float32, C-contiguous):

* ``means``          [3][N]   world-space centres (x, y, z planes)
* ``log_scales``     [3][N]   per-axis log standard deviations
* ``quats``          [4][N]   rotation quaternions (w, x, y, z planes)
* ``opacity_logits`` [N]      opacity before the logistic function
* ``sh``             [K*3][N] spherical-harmonic coefficients, plane k*3+c
                              holds basis function k of colour channel c,
                              K = (degree+1)^2

The Gaussian parameter set (mean, rotation + scale, opacity, SH colour) is
the one described in "Scaling 3D Gaussian Splatting with Distributed
Compute" (section "Where the Memory Goes") and in Splaxel, section 2.

Cameras are pinhole cameras with OpenCV axes (x right, y down, z forward);
``viewmat`` is the row-major 4x4 world-to-camera matrix.  The five workload
recipes follow the scene descriptions used for measurement: a 1K-Gaussian
64x64 scene, a 100K SH3 512x512 scene, a 1M clustered 1080p scene with four
views, a 10M skewed 4K scene and a 20M 4K scene split into four depth slabs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# SH degree-0 basis value 1/(2*sqrt(pi)).  Only used so that a degree-0 scene
# can be specified directly by its RGB colour (colour = coefficient * Y00).
_INV_Y00 = 2.0 * math.sqrt(math.pi)

FOV_X_DEG = 60.0


@dataclass
class Camera:
    viewmat: torch.Tensor          # float32 [16] row-major world->camera
    fx: float
    fy: float
    cx: float
    cy: float
    width: int
    height: int
    near_z: float = 0.01


@dataclass
class Scene:
    name: str
    sh_degree: int
    means: torch.Tensor
    log_scales: torch.Tensor
    quats: torch.Tensor
    opacity_logits: torch.Tensor
    sh: torch.Tensor
    cameras: list
    targets: list
    # depth slabs [lo, hi) of camera-space depth for partial renders
    depth_slabs: list = field(default_factory=list)
    adam: bool = True

    @property
    def n(self) -> int:
        return int(self.means.shape[1])

    @property
    def k_sh(self) -> int:
        return (self.sh_degree + 1) ** 2


def intrinsics(width: int, height: int, fov_x_deg: float = FOV_X_DEG):
    """Focal length from a horizontal field of view; principal point at the image centre."""
    f = (width / 2.0) / math.tan(math.radians(fov_x_deg) / 2.0)
    return f, f, width / 2.0, height / 2.0


def look_at_viewmat(position, target=(0.0, 0.0, 0.0), down=(0.0, 1.0, 0.0)) -> torch.Tensor:
    """World->camera matrix for a camera at ``position`` looking at ``target``.

    Camera axes: z forward (towards the target), x = normalise(down x z),
    y = z x x (so +y points roughly along ``down``).  If the view direction is
    nearly parallel to ``down``, world +z is used as the down hint instead.
    """
    pos = torch.tensor(position, dtype=torch.float64)
    tgt = torch.tensor(target, dtype=torch.float64)
    z = tgt - pos
    z = z / z.norm()
    d = torch.tensor(down, dtype=torch.float64)
    if abs(float(torch.dot(z, d / d.norm()))) > 0.99:
        d = torch.tensor((0.0, 0.0, 1.0), dtype=torch.float64)
    x = torch.linalg.cross(d, z)
    x = x / x.norm()
    y = torch.linalg.cross(z, x)
    R = torch.stack([x, y, z])               # rows = camera axes in world frame
    t = -R @ pos
    M = torch.eye(4, dtype=torch.float64)
    M[:3, :3] = R
    M[:3, 3] = t
    return M.reshape(16).to(torch.float32)


def _camera(viewmat, width, height):
    fx, fy, cx, cy = intrinsics(width, height)
    return Camera(viewmat=viewmat, fx=fx, fy=fy, cx=cx, cy=cy, width=width, height=height)


def _sphere_cameras(seed: int, count: int, radius: float, width: int, height: int):
    g = torch.Generator().manual_seed(seed)
    cams = []
    for _ in range(count):
        u = torch.randn(3, generator=g, dtype=torch.float32).double()
        u = u / u.norm()
        cams.append(_camera(look_at_viewmat(tuple((radius * u).tolist())), width, height))
    return cams


def _targets(seed: int, count: int, width: int, height: int):
    g = torch.Generator().manual_seed(seed)
    return [torch.rand(height, width, 3, generator=g, dtype=torch.float32) for _ in range(count)]


def _unit_quats(g, n):
    q = torch.randn(4, n, generator=g, dtype=torch.float32)
    return (q / q.norm(dim=0, keepdim=True)).contiguous()


def _sh_coeffs(g, n, degree, dc_uniform=True):
    k = (degree + 1) ** 2
    dc = torch.rand(3, n, generator=g, dtype=torch.float32)
    rest = 0.2 * torch.randn((k - 1) * 3, n, generator=g, dtype=torch.float32)
    return torch.cat([dc, rest], dim=0).contiguous()


def _random_rotations(g, count):
    """Uniformly random rotation matrices from the QR factorisation of Gaussian matrices."""
    a = torch.randn(count, 3, 3, generator=g, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    s = torch.sign(torch.diagonal(r, dim1=-2, dim2=-1))
    q = q * s.unsqueeze(-2)
    det = torch.linalg.det(q)
    q[det < 0, :, 0] *= -1.0
    return q


def _clustered_means(g, n, n_dense_clusters, n_sparse_clusters, dense_share, cube=20.0,
                     dense_volume_share=0.1):
    """Anisotropic Gaussian clusters: ``dense_share`` of the points sit in clusters whose
    centres lie in a central sub-cube holding ``dense_volume_share`` of the volume."""
    half = cube / 2.0
    sub_half = half * dense_volume_share ** (1.0 / 3.0)
    n_dense = int(round(n * dense_share))
    n_sparse = n - n_dense
    centres = torch.cat([
        (torch.rand(n_dense_clusters, 3, generator=g, dtype=torch.float64) * 2 - 1) * sub_half,
        (torch.rand(n_sparse_clusters, 3, generator=g, dtype=torch.float64) * 2 - 1) * half,
    ])
    ncl = n_dense_clusters + n_sparse_clusters
    counts = []
    for total, k in ((n_dense, n_dense_clusters), (n_sparse, n_sparse_clusters)):
        base, extra = divmod(total, k)
        counts += [base + (1 if i < extra else 0) for i in range(k)]
    log_lo, log_hi = math.log(0.05), math.log(1.0)
    sig = torch.exp(log_lo + (log_hi - log_lo) * torch.rand(ncl, 3, generator=g, dtype=torch.float64))
    rots = _random_rotations(g, ncl)
    out = torch.empty(n, 3, dtype=torch.float32)
    pos = 0
    for c in range(ncl):
        m = counts[c]
        z = torch.randn(m, 3, generator=g, dtype=torch.float64) * sig[c]
        out[pos:pos + m] = (z @ rots[c].T + centres[c]).to(torch.float32)
        pos += m
    return out.T.contiguous()


def _depth_slabs(means, viewmat, parts):
    """Camera-space depth boundaries splitting the Gaussians into ``parts`` slabs of
    (nearly) equal size; the first slab starts at 0 and the last ends at +inf."""
    M = viewmat.double().reshape(4, 4)
    z = (M[2, :3].unsqueeze(1) * means.double()).sum(0) + M[2, 3]
    zs = torch.sort(z).values
    n = zs.numel()
    bounds = [0.0]
    for k in range(1, parts):
        i = (k * n) // parts
        bounds.append(float(torch.tensor(0.5 * (zs[i - 1] + zs[i]).item(), dtype=torch.float32)))
    bounds.append(math.inf)
    return [(bounds[k], bounds[k + 1]) for k in range(parts)]


def slab_scenes(sc: Scene) -> list:
    """The scene's Gaussians split by its depth slabs into one scene per slab (camera-space
    depth of view 0 in double precision, window [lo, hi)); each keeps the cameras and
    targets.  Slabs are disjoint and ordered front to back."""
    M = sc.cameras[0].viewmat.double().reshape(4, 4)
    z = (M[2, :3].unsqueeze(1) * sc.means.double()).sum(0) + M[2, 3]
    out = []
    for k, (lo, hi) in enumerate(sc.depth_slabs):
        idx = torch.nonzero((z >= lo) & (z < hi)).squeeze(1)
        pick = lambda t: t[..., idx].contiguous()
        out.append(Scene(f"{sc.name}_slab{k}", sc.sh_degree, pick(sc.means), pick(sc.log_scales), pick(sc.quats),
                         pick(sc.opacity_logits), pick(sc.sh), sc.cameras, sc.targets, adam=sc.adam))
    return out


# --------------------------------------------------------------------------- configs

def scene_tiny(seed: int = 1) -> Scene:
    """1,024 Gaussians, SH degree 0 with RGB ~ U(0,1), means U[-1,1]^3, 64x64,
    camera at z=-3 looking along +z."""
    g = torch.Generator().manual_seed(seed)
    n = 1024
    means = (torch.rand(3, n, generator=g, dtype=torch.float32) * 2 - 1).contiguous()
    log_scales = (-3.0 + 0.5 * torch.randn(3, n, generator=g, dtype=torch.float32)).contiguous()
    quats = _unit_quats(g, n)
    logits = torch.randn(n, generator=g, dtype=torch.float32)
    rgb = torch.rand(3, n, generator=g, dtype=torch.float32)
    sh = (rgb * _INV_Y00).contiguous()
    vm = torch.eye(4, dtype=torch.float32)
    vm[2, 3] = 3.0
    cams = [_camera(vm.reshape(16).contiguous(), 64, 64)]
    return Scene("tiny_1k_64", 0, means, log_scales, quats, logits, sh, cams,
                 _targets(200 + seed, 1, 64, 64), adam=False)


def scene_100k(seed: int = 2) -> Scene:
    """100,000 Gaussians, SH3, means U[-5,5]^3, 512x512, camera at z=-15 looking along +z."""
    g = torch.Generator().manual_seed(seed)
    n = 100_000
    means = ((torch.rand(3, n, generator=g, dtype=torch.float32) * 2 - 1) * 5.0).contiguous()
    log_scales = (-4.0 + 0.5 * torch.randn(3, n, generator=g, dtype=torch.float32)).contiguous()
    quats = _unit_quats(g, n)
    logits = torch.randn(n, generator=g, dtype=torch.float32)
    sh = _sh_coeffs(g, n, 3)
    vm = torch.eye(4, dtype=torch.float32)
    vm[2, 3] = 15.0
    cams = [_camera(vm.reshape(16).contiguous(), 512, 512)]
    return Scene("sh3_100k_512", 3, means, log_scales, quats, logits, sh, cams,
                 _targets(200 + seed, 1, 512, 512))


def scene_1m_1080p(seed: int = 3, n: int = 1_000_000, views: int = 4) -> Scene:
    """1M Gaussians in 64 isotropic clusters (sigma 0.5 m) in a 20 m cube, SH3,
    1920x1080, cameras on a sphere of radius 25 looking at the origin."""
    g = torch.Generator().manual_seed(seed)
    ncl = 64
    centres = (torch.rand(ncl, 3, generator=g, dtype=torch.float64) * 2 - 1) * 10.0
    per = n // ncl
    counts = [per + (1 if i < n - per * ncl else 0) for i in range(ncl)]
    pts = torch.cat([centres[c] + 0.5 * torch.randn(counts[c], 3, generator=g, dtype=torch.float64)
                     for c in range(ncl)])
    means = pts.to(torch.float32).T.contiguous()
    log_scales = (-4.0 + 0.5 * torch.randn(3, n, generator=g, dtype=torch.float32)).contiguous()
    quats = _unit_quats(g, n)
    logits = torch.randn(n, generator=g, dtype=torch.float32)
    sh = _sh_coeffs(g, n, 3)
    cams = _sphere_cameras(100 + seed, views, 25.0, 1920, 1080)
    return Scene("sh3_1m_1080p", 3, means, log_scales, quats, logits, sh, cams,
                 _targets(200 + seed, views, 1920, 1080))


def scene_skewed_4k(seed: int = 4, n: int = 10_000_000, width: int = 3840, height: int = 2160,
                    slabs: int = 0) -> Scene:
    """Clustered 4K scene: 256 anisotropic clusters, 80% of the points in clusters whose
    centres lie in the central 10% of a 20 m cube; opacity logits N(1,1)."""
    g = torch.Generator().manual_seed(seed)
    n_dense_cl = 230
    means = _clustered_means(g, n, n_dense_cl, 256 - n_dense_cl, 0.8)
    log_scales = (-4.0 + 0.5 * torch.randn(3, n, generator=g, dtype=torch.float32)).contiguous()
    quats = _unit_quats(g, n)
    logits = (1.0 + torch.randn(n, generator=g, dtype=torch.float32)).contiguous()
    sh = _sh_coeffs(g, n, 3)
    cams = _sphere_cameras(100 + seed, 1, 25.0, width, height)
    sc = Scene(f"sh3_{n // 1_000_000}m_4k", 3, means, log_scales, quats, logits, sh, cams,
               _targets(200 + seed, 1, width, height))
    if slabs:
        sc.depth_slabs = _depth_slabs(means, cams[0].viewmat, slabs)
        sc.name += f"_{slabs}slabs"
    return sc


def scene_partitioned_4k(seed: int = 5, n: int = 20_000_000, width: int = 3840, height: int = 2160,
                         parts: int = 4) -> Scene:
    """20M Gaussians by the skewed recipe, split into ``parts`` depth-disjoint slabs."""
    return scene_skewed_4k(seed=seed, n=n, width=width, height=height, slabs=parts)


def scene_small_random(seed: int, n: int, width: int, height: int, sh_degree: int,
                       extent: float = 1.0, distance: float = 3.0, log_scale_mean: float = -2.5,
                       logit_mean: float = 0.0) -> Scene:
    """Small scenes for tests (ragged image sizes, any SH degree)."""
    g = torch.Generator().manual_seed(seed)
    means = ((torch.rand(3, n, generator=g, dtype=torch.float32) * 2 - 1) * extent).contiguous()
    log_scales = (log_scale_mean + 0.5 * torch.randn(3, n, generator=g, dtype=torch.float32)).contiguous()
    quats = _unit_quats(g, n)
    logits = (logit_mean + torch.randn(n, generator=g, dtype=torch.float32)).contiguous()
    sh = _sh_coeffs(g, n, sh_degree)
    vm = torch.eye(4, dtype=torch.float32)
    vm[2, 3] = distance
    cams = [_camera(vm.reshape(16).contiguous(), width, height)]
    return Scene(f"small_{n}_{width}x{height}_sh{sh_degree}", sh_degree, means, log_scales, quats,
                 logits, sh, cams, _targets(200 + seed, 1, width, height))


CONFIGS = {
    "tiny": scene_tiny,
    "100k": scene_100k,
    "1m": scene_1m_1080p,
    "10m": scene_skewed_4k,
    "20m": scene_partitioned_4k,
}


# --------------------------------------------------------------------------- synthetic stage inputs

def projected_for_binning(seed: int, n: int, width: int, height: int, cull_frac: float = 0.2,
                          max_radius: int = 40, dup_depth_frac: float = 0.1):
    """Synthetic projected records for testing the binning stage in isolation:
    pixel means inside the image, integer radii (0 marks a culled Gaussian) and
    positive float32 depths, with a share of exactly repeated depth values so
    that index tie-breaking is exercised."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(n, generator=g, dtype=torch.float32) * width
    v = torch.rand(n, generator=g, dtype=torch.float32) * height
    means2d = torch.stack([u, v], dim=1).contiguous()
    # heavy-tailed radii: most small, a few large
    r = torch.floor(torch.exp(torch.rand(n, 2, generator=g) * math.log(max_radius))).to(torch.int32)
    r = torch.clamp(r, min=1)
    culled = torch.rand(n, generator=g) < cull_frac
    r[culled] = 0
    depth = 0.5 + 50.0 * torch.rand(n, generator=g, dtype=torch.float32)
    dup = torch.rand(n, generator=g) < dup_depth_frac
    pool = 0.5 + 50.0 * torch.rand(16, generator=g, dtype=torch.float32)
    depth[dup] = pool[torch.randint(0, 16, (int(dup.sum()),), generator=g)]
    return means2d, r.contiguous(), depth.contiguous()


def sparse_grads(seed: int, n: int, zero_frac: float = 0.7, neg_zero_frac: float = 0.05):
    """[9][n] float32 gradients where ``zero_frac`` of the columns are all zero
    (some stored as -0.0) and the rest have at least one non-zero field."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(9, n, generator=g, dtype=torch.float32)
    zero_cols = torch.rand(n, generator=g) < zero_frac
    x[:, zero_cols] = 0.0
    negz = (torch.rand(9, n, generator=g) < neg_zero_frac) & zero_cols.unsqueeze(0)
    x[negz] = -0.0
    # partially zero columns among the non-zero ones
    part = (torch.rand(9, n, generator=g) < 0.5) & (~zero_cols).unsqueeze(0)
    keep = torch.randint(0, 9, (n,), generator=g)
    part[keep, torch.arange(n)] = False
    x[part] = 0.0
    return x.contiguous()


def adam_state(seed: int, n: int, step: int):
    """Parameters, gradients and Adam moments for an optimiser step."""
    g = torch.Generator().manual_seed(seed)
    p = torch.randn(n, generator=g, dtype=torch.float32)
    grad = torch.randn(n, generator=g, dtype=torch.float32) * 1e-3
    grad[torch.rand(n, generator=g) < 0.1] = 0.0
    if step <= 1:
        m = torch.zeros(n, dtype=torch.float32)
        v = torch.zeros(n, dtype=torch.float32)
    else:
        m = torch.randn(n, generator=g, dtype=torch.float32) * 1e-3
        v = torch.rand(n, generator=g, dtype=torch.float32) * 1e-6
    return p, grad, m, v


def partial_images(seed: int, parts: int, n_px: int, opaque_frac: float = 0.1):
    """Per-slab partial colours and transmittances in [0,1]; some pixels fully
    saturated (transmittance ~0) so that the saturation skip is exercised."""
    g = torch.Generator().manual_seed(seed)
    cs, ts = [], []
    for _ in range(parts):
        t = torch.rand(n_px, generator=g, dtype=torch.float32)
        t[torch.rand(n_px, generator=g) < opaque_frac] = 1e-6
        c = torch.rand(n_px, 3, generator=g, dtype=torch.float32) * (1 - t).unsqueeze(1)
        cs.append(c.contiguous())
        ts.append(t.contiguous())
    return cs, ts
