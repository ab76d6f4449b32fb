"""An independent float64 forward of the training step written with torch ops,
used only as a pin for the oracle's hand-written backward (torch.autograd
differentiates it).  Brute force: every pixel composites every Gaussian in
depth order.  Written from the same definitions as the oracle but sharing no
code with it:

* Sigma = R S S^T R^T, Sigma2D = J W Sigma W^T J^T, culling by the mean
  (Splaxel, section 2);
* front-to-back compositing with the alpha-check and termination at theta_T
  (ByteSplat, section 2.1, Eq. 1);
* colour from a real spherical-harmonic basis of degree <= 3 written out as
  Cartesian polynomials (textbook table, no Condon-Shortley phase).
"""
from __future__ import annotations

import math

import torch

# Real SH basis, degree <= 3, in Cartesian form on the unit sphere.
_C0 = 0.5 / math.sqrt(math.pi)
_C1 = math.sqrt(3.0 / (4.0 * math.pi))
_C2 = (math.sqrt(15.0 / math.pi) / 2.0, math.sqrt(5.0 / math.pi) / 4.0, math.sqrt(15.0 / math.pi) / 4.0)
_C3 = (math.sqrt(35.0 / (2.0 * math.pi)) / 4.0, math.sqrt(105.0 / math.pi) / 2.0,
       math.sqrt(21.0 / (2.0 * math.pi)) / 4.0, math.sqrt(7.0 / math.pi) / 4.0, math.sqrt(105.0 / math.pi) / 4.0)


def sh_poly(deg, x, y, z):
    out = [torch.full_like(x, _C0)]
    if deg >= 1:
        out += [_C1 * y, _C1 * z, _C1 * x]
    if deg >= 2:
        out += [_C2[0] * x * y, _C2[0] * y * z, _C2[1] * (3 * z * z - 1), _C2[0] * x * z,
                _C2[2] * (x * x - y * y)]
    if deg >= 3:
        out += [_C3[0] * y * (3 * x * x - y * y), _C3[1] * x * y * z, _C3[2] * y * (5 * z * z - 1),
                _C3[3] * z * (5 * z * z - 3), _C3[2] * x * (5 * z * z - 1), _C3[4] * z * (x * x - y * y),
                _C3[0] * x * (x * x - 3 * y * y)]
    return torch.stack(out, dim=0)          # [K][n]


def rot_from_quat(q):                        # q [4][n] unit, (w, x, y, z)
    w, x, y, z = q
    return torch.stack([
        torch.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)]),
        torch.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)]),
        torch.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]),
    ]).permute(2, 0, 1)                      # [n][3][3]


def forward(params, sh_degree, viewmat, fx, fy, cx, cy, width, height,
            alpha_min=1.0 / 255.0, alpha_max=0.99, t_min=1e-4, near_z=0.01):
    """params: dict of float64 tensors means [3][n], log_scales [3][n], quats [4][n],
    opacity_logits [n], sh [K*3][n].  Returns (color [H][W][3], T [H][W])."""
    mu = params["means"]
    n = mu.shape[1]
    s = torch.exp(params["log_scales"])
    q = params["quats"] / params["quats"].norm(dim=0, keepdim=True)
    o = torch.sigmoid(params["opacity_logits"])
    Rv = viewmat.reshape(4, 4)[:3, :3].double()
    tv = viewmat.reshape(4, 4)[:3, 3].double()
    p = Rv @ mu + tv[:, None]
    X, Y, Z = p
    u = fx * X / Z + cx
    v = fy * Y / Z + cy
    R = rot_from_quat(q)
    M = R * s.T[:, None, :]
    Sig = M @ M.transpose(1, 2)
    zero = torch.zeros_like(Z)
    J = torch.stack([torch.stack([fx / Z, zero, -fx * X / Z ** 2]),
                     torch.stack([zero, fy / Z, -fy * Y / Z ** 2])]).permute(2, 0, 1)
    T = J @ Rv
    S2 = T @ Sig @ T.transpose(1, 2)
    a, b, c = S2[:, 0, 0], 0.5 * (S2[:, 0, 1] + S2[:, 1, 0]), S2[:, 1, 1]
    det = a * c - b * b
    A, B, C = c / det, -b / det, a / det
    campos = -Rv.T @ tv
    d = mu - campos[:, None]
    d = d / d.norm(dim=0, keepdim=True)
    Ysh = sh_poly(sh_degree, d[0], d[1], d[2])          # [K][n]
    K = Ysh.shape[0]
    shc = params["sh"].reshape(K, 3, n)
    col = (shc * Ysh[:, None, :]).sum(0)                  # [3][n]

    vis = (Z > near_z) & (u >= 0) & (u < width) & (v >= 0) & (v < height) & (det > 0) & (o >= alpha_min)
    Zd = Z.detach()
    order = sorted([i for i in range(n) if bool(vis[i])], key=lambda i: (float(Zd[i]), i))

    ys, xs = torch.meshgrid(torch.arange(height, dtype=torch.float64),
                            torch.arange(width, dtype=torch.float64), indexing="ij")
    px, py = xs + 0.5, ys + 0.5
    Tm = torch.ones(height, width, dtype=torch.float64)
    img = torch.zeros(height, width, 3, dtype=torch.float64)
    for i in order:
        dx, dy = px - u[i], py - v[i]
        power = -0.5 * (A[i] * dx * dx + C[i] * dy * dy) - B[i] * dx * dy
        raw = o[i] * torch.exp(power)
        alpha = torch.minimum(raw, torch.tensor(alpha_max, dtype=torch.float64))
        live = (Tm.detach() >= t_min) & (alpha.detach() >= alpha_min)
        w = torch.where(live, Tm * alpha, torch.zeros_like(alpha))
        img = img + w[..., None] * col[:, i]
        Tm = torch.where(live, Tm * (1 - alpha), Tm)
    return img, Tm
