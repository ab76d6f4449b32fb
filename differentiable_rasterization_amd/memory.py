"""Memory planning for one GPU (MI355X: 288 GB of HBM3E).

Per-Gaussian float32 scalars: mean 3, scale 3 + quaternion 4, opacity 1, SH
3*(degree+1)^2 ("Scaling 3D Gaussian Splatting with Distributed Compute",
section "Where the Memory Goes": 38 learnable scalars and 456 bytes with the
two Adam moments at SH degree 2, 59 scalars and about 708 bytes at degree 3).
This library adds the gradient copy, the projected record, the screen-space
gradients and the binning workspace; those are counted separately.
"""
from __future__ import annotations

MI355X_HBM_BYTES = 288e9


def learnable_scalars(sh_degree: int) -> int:
    return 3 + 3 + 4 + 1 + 3 * (sh_degree + 1) ** 2


def bytes_per_gaussian(sh_degree: int, adam: bool = True, grads: bool = False) -> int:
    """Parameters (+ Adam moments) (+ a gradient copy), float32."""
    copies = 1 + (2 if adam else 0) + (1 if grads else 0)
    return 4 * learnable_scalars(sh_degree) * copies


def step_bytes_per_gaussian(sh_degree: int) -> int:
    """Everything this library keeps per Gaussian during a training step: parameters,
    gradients, Adam moments, the projection's depth key (4), radii (8) and 48-byte raster
    record (the plain record planes are optional and not counted), screen-space gradients
    (36), the binning's per-Gaussian buffers (36: 32-bit depth keys and 64-bit values (tile
    count, index) twice, quadrant-record counts, emit offsets, first gradient slot) and the
    raster buffer's per-Gaussian part (68: the record copied at a 64-byte stride, the first
    gradient slot)."""
    return bytes_per_gaussian(sh_degree, adam=True, grads=True) + 60 + 36 + 36 + 68


def step_bytes_per_intersection() -> int:
    """Intersection lists: ids (4); the raster lists with room for two 8x8-quadrant entries
    per tile entry (2 x 12: Gaussian, gradient slot, tile-list position), their gradient
    slots (2 x 48) and slot stamps (2 x 4), and 4 quadrant bits (0.5, counted as 1); and the
    sort workspace's key, value, Gaussian and first-slot buffers (24)."""
    return 4 + 2 * (12 + 48 + 4) + 1 + 24


def max_gaussians(hbm_bytes: float, sh_degree: int, adam: bool = True) -> int:
    return int(hbm_bytes // bytes_per_gaussian(sh_degree, adam=adam))


def max_gaussians_training(hbm_bytes: float, sh_degree: int, intersections_per_gaussian: float) -> int:
    per = step_bytes_per_gaussian(sh_degree) + intersections_per_gaussian * step_bytes_per_intersection()
    return int(hbm_bytes // per)
