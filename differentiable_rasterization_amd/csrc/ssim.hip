// The objective with its structural term (ROCm blog, "Why gsplat Cannot Just Use DDP":
// L = (1 - lambda) mean |C - C*| + lambda (1 - SSIM(C, C*)) / 2; Splaxel section 2
// "Parameter Optimization"; ByteSplat Eq. 2), and its gradient dL/dC.
//
// SSIM per colour channel with an 11 x 11 Gaussian window (sigma 1.5, normalised over its
// support), zero padding outside the image, C1 = 0.01^2, C2 = 0.03^2; SSIM = the mean of
// the per-pixel index S over the pixels and channels.  At pixel p, with window sums
// mu_x = G*x, mu_y = G*y, e_xx = G*x^2, e_yy = G*y^2, e_xy = G*(x y):
//   S = (2 mu_x mu_y + C1)(2 s_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(s_xx + s_yy + C2)),
//   s_xx = e_xx - mu_x^2, s_yy = e_yy - mu_y^2, s_xy = e_xy - mu_x mu_y.
// Its gradient with respect to x at pixel q goes through every window that holds q:
//   dSSIM/dx(q) = (1/N) [ (G*a)(q) + 2 x(q) (G*b)(q) + y(q) (G*c)(q) ],
//   a = dS/dmu_x (through s_xx and s_xy too), b = dS/de_xx, c = dS/de_xy per pixel p,
// N = 3 H W, G symmetric.  Two kernels: k_ssim_maps forms the window sums and the three
// coefficient maps a, b, c (and the block's sums of S and |C - C*|); k_ssim_grad filters
// the maps with the same window and combines them with x, y and the L1 term into dL/dC.
// Both are separable 11-tap filters over 64 x 16 output tiles staged in LDS with a
// 5-pixel halo (zero outside the image).
#include <cmath>

#include "kernels.h"

namespace {

constexpr int kR = 5, kTaps = 2 * kR + 1;
constexpr int kTW = 64, kTH = 16;                       // output tile
constexpr int kRW = kTW + 2 * kR, kRH = kTH + 2 * kR;   // tile + halo: 74 x 26
constexpr int kThreads = 256;
constexpr float kC1 = 1e-4f, kC2 = 9e-4f;

struct Window {
    float g[kTaps];
};

// Per block: sum of S and of |C - C*| over its output pixels and channels.
struct SsimPartial {
    double s, l1;
};

__global__ __launch_bounds__(kThreads) void k_ssim_maps(const float *__restrict__ x, const float *__restrict__ y,
                                                        int W, int H, Window win, float *__restrict__ maps,
                                                        SsimPartial *__restrict__ part)
{
    // the tile + halo of both images, all three channels interleaved as in memory
    __shared__ float sx[kRH][kRW * 3], sy[kRH][kRW * 3];
    // horizontal window sums of mu_x, mu_y, e_xx, e_yy, e_xy over the tile's columns
    __shared__ float hs[5][kRH][kTW];
    __shared__ double red[2][kThreads / 64];
    const int t = threadIdx.x;
    const int x0 = blockIdx.x * kTW, y0 = blockIdx.y * kTH;
    for (int i = t; i < kRH * kRW * 3; i += kThreads) {
        const int r = i / (kRW * 3), k = i - r * (kRW * 3);
        const int gy = y0 - kR + r, gx = x0 - kR + k / 3;
        float a = 0.0f, b = 0.0f;
        if (gy >= 0 && gy < H && gx >= 0 && gx < W) {
            const size_t o = ((size_t)gy * W + gx) * 3 + (k % 3);
            a = x[o];
            b = y[o];
        }
        sx[r][k] = a;
        sy[r][k] = b;
    }
    __syncthreads();
    const size_t plane = (size_t)W * H;
    double s_acc = 0.0, l1_acc = 0.0;
    for (int c = 0; c < 3; ++c) {
        for (int i = t; i < kRH * kTW; i += kThreads) {
            const int r = i / kTW, col = i - r * kTW;
            float mx = 0.0f, my = 0.0f, exx = 0.0f, eyy = 0.0f, exy = 0.0f;
#pragma unroll
            for (int u = 0; u < kTaps; ++u) {
                const float a = sx[r][(col + u) * 3 + c], b = sy[r][(col + u) * 3 + c], w = win.g[u];
                const float wa = w * a, wb = w * b;
                mx += wa;
                my += wb;
                exx = fmaf(wa, a, exx);
                eyy = fmaf(wb, b, eyy);
                exy = fmaf(wa, b, exy);
            }
            hs[0][r][col] = mx;
            hs[1][r][col] = my;
            hs[2][r][col] = exx;
            hs[3][r][col] = eyy;
            hs[4][r][col] = exy;
        }
        __syncthreads();
        for (int i = t; i < kTH * kTW; i += kThreads) {
            const int r = i / kTW, col = i - r * kTW;
            const int gy = y0 + r, gx = x0 + col;
            float mx = 0.0f, my = 0.0f, exx = 0.0f, eyy = 0.0f, exy = 0.0f;
#pragma unroll
            for (int v = 0; v < kTaps; ++v) {
                const float w = win.g[v];
                mx = fmaf(w, hs[0][r + v][col], mx);
                my = fmaf(w, hs[1][r + v][col], my);
                exx = fmaf(w, hs[2][r + v][col], exx);
                eyy = fmaf(w, hs[3][r + v][col], eyy);
                exy = fmaf(w, hs[4][r + v][col], exy);
            }
            if (gy < H && gx < W) {
                const float sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
                const float n1 = 2.0f * mx * my + kC1, n2 = 2.0f * sxy + kC2;
                const float d1 = mx * mx + my * my + kC1, d2 = sxx + syy + kC2;
                const float S = (n1 * n2) / (d1 * d2);
                const float dS_dmx = S * (2.0f * my / n1 - 2.0f * mx / d1);
                const float dS_dsxx = -S / d2, dS_dsxy = 2.0f * S / n2;
                const size_t p = (size_t)gy * W + gx;
                maps[(size_t)(0 * 3 + c) * plane + p] = dS_dmx - 2.0f * mx * dS_dsxx - my * dS_dsxy;
                maps[(size_t)(1 * 3 + c) * plane + p] = dS_dsxx;
                maps[(size_t)(2 * 3 + c) * plane + p] = dS_dsxy;
                s_acc += (double)S;
                l1_acc += (double)fabsf(sx[r + kR][(col + kR) * 3 + c] - sy[r + kR][(col + kR) * 3 + c]);
            }
        }
        __syncthreads();
    }
    // block sums in a fixed order: each wave's butterfly, then the waves in order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s_acc += __shfl_xor(s_acc, o, 64);
        l1_acc += __shfl_xor(l1_acc, o, 64);
    }
    if ((t & 63) == 0) {
        red[0][t >> 6] = s_acc;
        red[1][t >> 6] = l1_acc;
    }
    __syncthreads();
    if (t == 0) {
        const int b = blockIdx.y * gridDim.x + blockIdx.x;
        part[b].s = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        part[b].l1 = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    }
}

// The loss and SSIM from the block sums (one block; each thread a strided share, then a
// fixed tree).
__global__ __launch_bounds__(kThreads) void k_ssim_final(const SsimPartial *__restrict__ part, int nb, double inv_n,
                                                         double lambda, float *__restrict__ loss,
                                                         float *__restrict__ ssim)
{
    __shared__ double red[2][kThreads / 64];
    const int t = threadIdx.x;
    double s = 0.0, l1 = 0.0;
    for (int b = t; b < nb; b += kThreads) {
        s += part[b].s;
        l1 += part[b].l1;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s += __shfl_xor(s, o, 64);
        l1 += __shfl_xor(l1, o, 64);
    }
    if ((t & 63) == 0) {
        red[0][t >> 6] = s;
        red[1][t >> 6] = l1;
    }
    __syncthreads();
    if (t == 0) {
        const double S = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) * inv_n;
        const double L1 = ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) * inv_n;
        if (loss) *loss = (float)((1.0 - lambda) * L1 + lambda * (1.0 - S) * 0.5);
        if (ssim) *ssim = (float)S;
    }
}

__global__ __launch_bounds__(kThreads) void k_ssim_grad(const float *__restrict__ x, const float *__restrict__ y,
                                                        int W, int H, Window win, const float *__restrict__ maps,
                                                        float w_l1, float w_ssim, float *__restrict__ dL_dc)
{
    __shared__ float sm[3][kRH][kRW];
    __shared__ float hs[3][kRH][kTW];
    const int t = threadIdx.x;
    const int x0 = blockIdx.x * kTW, y0 = blockIdx.y * kTH;
    const size_t plane = (size_t)W * H;
    for (int c = 0; c < 3; ++c) {
        for (int i = t; i < 3 * kRH * kRW; i += kThreads) {
            const int m = i / (kRH * kRW), rem = i - m * (kRH * kRW);
            const int r = rem / kRW, k = rem - r * kRW;
            const int gy = y0 - kR + r, gx = x0 - kR + k;
            float v = 0.0f;   // no window centred outside the image contributes
            if (gy >= 0 && gy < H && gx >= 0 && gx < W) v = maps[(size_t)(m * 3 + c) * plane + (size_t)gy * W + gx];
            sm[m][r][k] = v;
        }
        __syncthreads();
        for (int i = t; i < kRH * kTW; i += kThreads) {
            const int r = i / kTW, col = i - r * kTW;
            float a = 0.0f, b = 0.0f, cc = 0.0f;
#pragma unroll
            for (int u = 0; u < kTaps; ++u) {
                const float w = win.g[u];
                a = fmaf(w, sm[0][r][col + u], a);
                b = fmaf(w, sm[1][r][col + u], b);
                cc = fmaf(w, sm[2][r][col + u], cc);
            }
            hs[0][r][col] = a;
            hs[1][r][col] = b;
            hs[2][r][col] = cc;
        }
        __syncthreads();
        for (int i = t; i < kTH * kTW; i += kThreads) {
            const int r = i / kTW, col = i - r * kTW;
            const int gy = y0 + r, gx = x0 + col;
            if (gy >= H || gx >= W) continue;
            float a = 0.0f, b = 0.0f, cc = 0.0f;
#pragma unroll
            for (int v = 0; v < kTaps; ++v) {
                const float w = win.g[v];
                a = fmaf(w, hs[0][r + v][col], a);
                b = fmaf(w, hs[1][r + v][col], b);
                cc = fmaf(w, hs[2][r + v][col], cc);
            }
            const size_t o = ((size_t)gy * W + gx) * 3 + c;
            const float xv = x[o], yv = y[o];
            const float d = xv - yv;
            const float sg = d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f);
            const float gs = fmaf(2.0f * xv, b, fmaf(yv, cc, a));   // N dSSIM/dx
            dL_dc[o] = fmaf(w_l1, sg, -w_ssim * gs);
        }
        __syncthreads();
    }
}

struct SsimWs {
    size_t maps, part, bytes;
    int gx, gy;
};

SsimWs ssim_ws(int32_t W, int32_t H)
{
    SsimWs w;
    w.gx = (int)gsi::ceil_div(W, kTW);
    w.gy = (int)gsi::ceil_div(H, kTH);
    w.maps = 0;
    w.part = (size_t)9 * W * H * sizeof(float);
    w.part = (w.part + 255) & ~size_t(255);
    w.bytes = w.part + (size_t)w.gx * w.gy * sizeof(SsimPartial);
    return w;
}

}  // namespace

extern "C" size_t gs_loss_l1_dssim_workspace_bytes(int32_t width, int32_t height)
{
    if (width <= 0 || height <= 0 || width > 65536 || height > 65536) return 0;
    return ssim_ws(width, height).bytes;
}

extern "C" gs_status gs_loss_l1_dssim(const float *color, const float *target, int32_t width, int32_t height,
                                      float lambda, float *loss_out, float *ssim_out, float *dL_dcolor,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    using namespace gsi;
    if (width <= 0 || height <= 0 || width > 65536 || height > 65536)
        return fail(GS_ERR_INVALID_ARGUMENT, "image size %d x %d outside 1 .. 65536", width, height);
    if (!color || !target || !dL_dcolor) return fail(GS_ERR_INVALID_ARGUMENT, "color / target / dL_dcolor is NULL");
    if (!(lambda >= 0.0f && lambda <= 1.0f)) return fail(GS_ERR_INVALID_ARGUMENT, "lambda must lie in [0, 1]");
    const SsimWs ws = ssim_ws(width, height);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < ws.bytes)
        return fail(GS_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, 256-byte aligned", ws.bytes);
    Window win;
    {
        double g[kTaps], sum = 0.0;
        for (int u = -kR; u <= kR; ++u) sum += (g[u + kR] = std::exp(-(double)(u * u) / (2.0 * 1.5 * 1.5)));
        for (int u = 0; u < kTaps; ++u) win.g[u] = (float)(g[u] / sum);
    }
    char *wb = static_cast<char *>(workspace);
    float *maps = reinterpret_cast<float *>(wb + ws.maps);
    SsimPartial *part = reinterpret_cast<SsimPartial *>(wb + ws.part);
    const dim3 grid((unsigned)ws.gx, (unsigned)ws.gy);
    k_ssim_maps<<<grid, kThreads, 0, stream>>>(color, target, width, height, win, maps, part);
    GS_LAUNCH_CHECK("k_ssim_maps");
    const double n = 3.0 * (double)width * (double)height;
    k_ssim_final<<<1, kThreads, 0, stream>>>(part, ws.gx * ws.gy, 1.0 / n, (double)lambda, loss_out, ssim_out);
    GS_LAUNCH_CHECK("k_ssim_final");
    k_ssim_grad<<<grid, kThreads, 0, stream>>>(color, target, width, height, win, maps,
                                               (float)((1.0 - (double)lambda) / n), (float)(0.5 * (double)lambda / n),
                                               dL_dcolor);
    GS_LAUNCH_CHECK("k_ssim_grad");
    return GS_OK;
}
