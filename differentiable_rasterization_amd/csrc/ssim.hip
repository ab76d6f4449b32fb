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
// N = 3 H W, G symmetric.  k_ssim_maps forms the window sums and the three coefficient
// maps a, b, c (and the block's sum of S); k_ssim_grad filters the maps with the same
// window and combines them with x, y and the L1 term into dL/dC (and the block's sum of
// |C - C*|); k_ssim_final adds the block sums into the loss and SSIM.
// Both work on 64 x 16 output tiles, one channel at a time: the channel's tile with a
// 5-pixel halo (zero outside the image) is staged in LDS, filtered down the columns first
// (a lane takes four output rows of one of the first 64 columns, and one output of the 10
// remaining halo columns), then along the rows (four adjacent outputs per thread).  The
// next channel's loads are in flight meanwhile.
#include <cmath>

#include "kernels.h"

namespace {

constexpr int kR = 5, kTaps = 2 * kR + 1;
constexpr int kTW = 64, kTH = 16;                       // output tile
constexpr int kRW = kTW + 2 * kR, kRH = kTH + 2 * kR;   // tile + halo: 74 x 26
constexpr int kVW = kRW + 2;                            // row stride of the column sums (16-byte rows)
constexpr int kThreads = 256;
constexpr float kC1 = 1e-4f, kC2 = 9e-4f;
static_assert(kTW == 4 * (kThreads / kTH), "row pass: four outputs per thread");

struct Window {
    float g[kTaps];
};

// Per block: sum of S and of |C - C*| over its output pixels and channels.
struct SsimPartial {
    double s, l1;
};

// The staged loads of one channel of NP planes (tile + halo, zero outside the image).
// Plane m of channel c at pixel (gx, gy) is at base[m] + (gy W + gx) cs + coff.  Columns
// 0 .. 63 of the halo'd tile: lane = column, rows wave + 4k (wave-uniform); columns 64 .. 73:
// lanes 0 .. 59 of each wave take 6 rows of 10.  Every load is issued unconditionally (at
// offset 0 where the pixel is outside the image) and its value selected.
constexpr int kWaves = kThreads / 64;
constexpr int kSA = (kRH + kWaves - 1) / kWaves;                          // 7
constexpr int kBW = kRW - 64, kBL = 60;                                   // 10 columns, 60 lanes
constexpr int kSB = (kRH * kBW + kWaves * kBL - 1) / (kWaves * kBL);      // 2
static_assert(kRW > 64 && kRW <= 64 + kBW && kBL % kBW == 0, "halo layout");
// LDS row strides of the staged tiles are 16 mod 32 words, so that the two rows one paired
// read (ds_read2) fetches for a lane fall in different banks
constexpr int kRW3 = 3 * kRW, kRW3P = 240;                                // 222 floats per row
constexpr int kRWP = 80;                                                  // 74 floats per row
static_assert(kRW3P >= kRW3 && kRW3P % 32 == 16 && kRWP >= kRW && kRWP % 32 == 16, "LDS row strides");
constexpr int kSN3 = (kRH * kRW3 + kThreads - 1) / kThreads;              // 23
static_assert(kThreads >= kRW3 && kThreads < 2 * kRW3, "staging steps rows by one or two");
constexpr int kVR = kTH / kWaves;            // column pass: output rows per lane (4)
constexpr int kVB = kTH * kBW / kWaves;      // column pass: outputs of columns 64 .. 73 per wave (40)
static_assert(kVR * kWaves == kTH && kVB <= 64, "column pass layout");

template <int NP>
struct Stage {
    float a[NP][kSA], b[NP][kSB];
};

// A thread's staging positions, fixed for the block: pixel index (gy W + gx) of each of its
// kSA + kSB staged pixels, 0 where the pixel is outside the image (ok bit clear).
struct StagePos {
    uint32_t pix[kSA + kSB];
    uint32_t ok;   // bit k: pixel k inside the image
};

__device__ __forceinline__ void stage_b_pos(int k, int &r, int &col, bool &in)
{
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e = kBL * w + lane + kWaves * kBL * k;
    in = lane < kBL && e < kRH * kBW;
    r = e / kBW;
    col = 64 + (e - r * kBW);
}

__device__ __forceinline__ StagePos stage_pos(int W, int H, int x0, int y0)
{
    StagePos P;
    P.ok = 0u;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gxa = x0 - kR + lane;
    const bool col_ok = gxa >= 0 && gxa < W;
#pragma unroll
    for (int k = 0; k < kSA; ++k) {
        const int r = w + kWaves * k, gy = y0 - kR + r;
        const bool ok = col_ok && r < kRH && gy >= 0 && gy < H;
        P.pix[k] = ok ? (uint32_t)gy * (uint32_t)W + (uint32_t)gxa : 0u;
        P.ok |= ok ? 1u << k : 0u;
    }
#pragma unroll
    for (int k = 0; k < kSB; ++k) {
        int r, col;
        bool in;
        stage_b_pos(k, r, col, in);
        const int gy = y0 - kR + r, gx = x0 - kR + col;   // gx >= 59
        const bool ok = in && gy >= 0 && gy < H && gx < W;
        P.pix[kSA + k] = ok ? (uint32_t)gy * (uint32_t)W + (uint32_t)gx : 0u;
        P.ok |= ok ? 1u << (kSA + k) : 0u;
    }
    return P;
}

// Plane m's value at staged pixel k is at byte base[m] + pix[k] * bs (32-bit byte offsets:
// the caller keeps every offset below 2^32).
template <int NP>
__device__ __forceinline__ void stage_load(Stage<NP> &st, const StagePos &P, const char *const (&base)[NP],
                                           uint32_t bs)
{
#pragma unroll
    for (int k = 0; k < kSA + kSB; ++k) {
        const uint32_t off = P.pix[k] * bs;
        const bool ok = (P.ok >> k) & 1u;
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            const float v = *reinterpret_cast<const float *>(base[m] + off);
            if (k < kSA)
                st.a[m][k] = ok ? v : 0.0f;
            else
                st.b[m][k - kSA] = ok ? v : 0.0f;
        }
    }
}

template <int NP>
__device__ __forceinline__ void stage_store(const Stage<NP> &st, float (*sin)[kRH][kRWP])
{
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int k = 0; k < kSA; ++k) {
        const int r = w + kWaves * k;
        if (r < kRH) {
#pragma unroll
            for (int m = 0; m < NP; ++m) sin[m][r][lane] = st.a[m][k];
        }
    }
#pragma unroll
    for (int k = 0; k < kSB; ++k) {
        int r, col;
        bool in;
        stage_b_pos(k, r, col, in);
        if (in) {
#pragma unroll
            for (int m = 0; m < NP; ++m) sin[m][r][col] = st.b[m][k];
        }
    }
}

// Along the rows: the 14 column sums at row `row`, columns c4 .. c4 + 13 (c4 a multiple of
// 4), and from them out[j] = sum_u g[u] v[j + u] over a thread's four adjacent outputs.
__device__ __forceinline__ void row_load14(const float *__restrict__ rowp, float (&v)[16])
{
    *reinterpret_cast<float4 *>(&v[0]) = *reinterpret_cast<const float4 *>(rowp);
    *reinterpret_cast<float4 *>(&v[4]) = *reinterpret_cast<const float4 *>(rowp + 4);
    *reinterpret_cast<float4 *>(&v[8]) = *reinterpret_cast<const float4 *>(rowp + 8);
    *reinterpret_cast<float2 *>(&v[12]) = *reinterpret_cast<const float2 *>(rowp + 12);
}

__device__ __forceinline__ void row_filter4(const float (&v)[16], const Window &win, float (&out)[4])
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int u = 0; u < kTaps; ++u) a = fmaf(win.g[u], v[j + u], a);
        out[j] = a;
    }
}

// A block's sum of v in a fixed order (each wave's butterfly, then the waves in order),
// written by thread 0 to *out.
__device__ __forceinline__ void block_sum(double v, double (&red)[kThreads / 64], double *out)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) *out = (red[0] + red[1]) + (red[2] + red[3]);
}

// The tile a block takes: blocks reach the 8 XCDs round-robin (block b on XCD b % 8), and
// each XCD takes one contiguous run of the row-major tiles, so the halos that neighbouring
// tiles share are read through one L2.
__device__ __forceinline__ int xcd_tile(int tiles)
{
    const int b = blockIdx.x, xc = b % gsi::kXcds, per = tiles / gsi::kXcds, rem = tiles % gsi::kXcds;
    return xc * per + min(xc, rem) + b / gsi::kXcds;
}

__global__ __launch_bounds__(kThreads, 2) void k_ssim_maps(const float *__restrict__ x, const float *__restrict__ y,
                                                           int W, int H, Window win, float *__restrict__ maps,
                                                           SsimPartial *__restrict__ part, int tiles_x, int tiles)
{
    // the tile + halo of both images, all three channels interleaved as in memory (each
    // line of the images is read once)
    __shared__ float sin[2][kRH][kRW3P];
    // one channel's window sums down the columns: mu_x, mu_y, e_xx, e_yy, e_xy at the tile's rows
    __shared__ __align__(16) float sv[5][kTH][kVW];
    __shared__ double red[kThreads / 64];
    const int t = threadIdx.x;
    const int tile = xcd_tile(tiles);
    const int x0 = (tile % tiles_x) * kTW, y0 = (tile / tiles_x) * kTH;
    const size_t plane = (size_t)W * H;
    {   // row r of the staged tile: floats (gy W + x0 - 5) 3 .. + 222 of each image, of which
        // floats lo .. hi lie inside the image; element i = t + 256 k is (r, f), stepped
        // without division (256 = 222 + 34)
        const int lo = max(0, kR - x0) * 3, hi = min(kRW, W - x0 + kR) * 3;
        const uint32_t W3 = 3u * (uint32_t)W;
        float va[kSN3], vb[kSN3];
        {
            int r = t >= kRW3 ? 1 : 0, f = t - r * kRW3;
            uint32_t roff = ((uint32_t)(y0 - kR + r) * (uint32_t)W + (uint32_t)(x0 - kR)) * 3u;   // wraps: unused then
#pragma unroll
            for (int k = 0; k < kSN3; ++k) {
                const int gy = y0 - kR + r;
                const bool ok = r < kRH && gy >= 0 && gy < H && f >= lo && f < hi;
                const uint32_t off = ok ? roff + (uint32_t)f : 0u;
                const float a = x[off], b = y[off];
                va[k] = ok ? a : 0.0f;
                vb[k] = ok ? b : 0.0f;
                f += kThreads - kRW3;
                r += 1;
                roff += W3;
                if (f >= kRW3) {
                    f -= kRW3;
                    r += 1;
                    roff += W3;
                }
            }
        }
        int r = t >= kRW3 ? 1 : 0, f = t - r * kRW3;
#pragma unroll
        for (int k = 0; k < kSN3; ++k) {
            if (r < kRH) {
                sin[0][r][f] = va[k];
                sin[1][r][f] = vb[k];
            }
            f += kThreads - kRW3;
            r += 1;
            if (f >= kRW3) {
                f -= kRW3;
                r += 1;
            }
        }
    }
    const int hr = t / (kTW / 4), c4 = 4 * (t % (kTW / 4));   // row pass: row, first column
    const int gy = y0 + hr;
    // column pass: lane = column 0 .. 63 at rows vr0 .. vr0 + 3; lanes 0 .. 39 of each wave
    // also take one of the 160 outputs of columns 64 .. 73
    const int lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6), vr0 = kVR * wv;
    const int vb_e = kVB * wv + lane, vb_r = vb_e / kBW, vb_c = 64 + (vb_e - vb_r * kBW);
    const bool vb_in = lane < kVB;
    double s_acc = 0.0;
    for (int c = 0; c < 3; ++c) {
        __syncthreads();   // sin is staged; sv is free
        {   // columns 0 .. 63: lane = column, rows 4 w .. 4 w + 3 (14 input rows)
            float acc[5][kVR];
#pragma unroll
            for (int q = 0; q < 5; ++q)
#pragma unroll
                for (int j = 0; j < kVR; ++j) acc[q][j] = 0.0f;
            float ca[kVR + 2 * kR], cb[kVR + 2 * kR];   // all reads issued before the first use
#pragma unroll
            for (int i = 0; i < kVR + 2 * kR; ++i) {
                ca[i] = sin[0][vr0 + i][3 * lane + c];
                cb[i] = sin[1][vr0 + i][3 * lane + c];
            }
#pragma unroll
            for (int i = 0; i < kVR + 2 * kR; ++i) {
                const float a = ca[i], b = cb[i];
                const float v[5] = {a, b, a * a, b * b, a * b};
#pragma unroll
                for (int j = 0; j < kVR; ++j)
                    if (i - j >= 0 && i - j < kTaps)
#pragma unroll
                        for (int q = 0; q < 5; ++q) acc[q][j] = fmaf(win.g[i - j], v[q], acc[q][j]);
            }
#pragma unroll
            for (int q = 0; q < 5; ++q)
#pragma unroll
                for (int j = 0; j < kVR; ++j) sv[q][vr0 + j][lane] = acc[q][j];
        }
        if (vb_in) {   // columns 64 .. 73: one output per lane
            float acc[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            float ca[kTaps], cb[kTaps];
#pragma unroll
            for (int u = 0; u < kTaps; ++u) {
                ca[u] = sin[0][vb_r + u][3 * vb_c + c];
                cb[u] = sin[1][vb_r + u][3 * vb_c + c];
            }
#pragma unroll
            for (int u = 0; u < kTaps; ++u) {
                const float a = ca[u], b = cb[u];
                const float v[5] = {a, b, a * a, b * b, a * b};
#pragma unroll
                for (int q = 0; q < 5; ++q) acc[q] = fmaf(win.g[u], v[q], acc[q]);
            }
#pragma unroll
            for (int q = 0; q < 5; ++q) sv[q][vb_r][vb_c] = acc[q];
        }
        __syncthreads();   // sv holds channel c
        float rv[5][16];   // all reads issued before the first use
#pragma unroll
        for (int q = 0; q < 5; ++q) row_load14(&sv[q][hr][c4], rv[q]);
        float mx[4], my[4], exx[4], eyy[4], exy[4];
        row_filter4(rv[0], win, mx);
        row_filter4(rv[1], win, my);
        row_filter4(rv[2], win, exx);
        row_filter4(rv[3], win, eyy);
        row_filter4(rv[4], win, exy);
        float ma[4], mb[4], mc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // S = n1 n2 / (d1 d2); its derivatives written without dividing by n1 or n2
            const float sxx = exx[j] - mx[j] * mx[j], syy = eyy[j] - my[j] * my[j], sxy = exy[j] - mx[j] * my[j];
            const float n1 = 2.0f * mx[j] * my[j] + kC1, n2 = 2.0f * sxy + kC2;
            const float d1 = mx[j] * mx[j] + my[j] * my[j] + kC1, d2 = sxx + syy + kC2;   // d1 >= C1, d2 ~ >= C2
            const float i1 = __builtin_amdgcn_rcpf(d1), i2 = __builtin_amdgcn_rcpf(d2), D = i1 * i2;   // 1 ulp
            const float S = n1 * n2 * D;
            const float dS_dmx = 2.0f * (my[j] * n2 * D - mx[j] * S * i1);
            const float dS_dsxx = -S * i2, dS_dsxy = 2.0f * n1 * D;
            ma[j] = dS_dmx - 2.0f * mx[j] * dS_dsxx - my[j] * dS_dsxy;
            mb[j] = dS_dsxx;
            mc[j] = dS_dsxy;
            if (gy < H && x0 + c4 + j < W) s_acc += (double)S;
        }
        if (gy < H) {
            const int gx = x0 + c4;
            const size_t p = (size_t)gy * W + gx;
            float *m0 = maps + (size_t)c * plane + p, *m1 = maps + (size_t)(3 + c) * plane + p,
                  *m2 = maps + (size_t)(6 + c) * plane + p;
            if (gx + 3 < W && ((p | plane) & 3) == 0) {   // the three planes' rows 16-byte aligned
                *reinterpret_cast<float4 *>(m0) = make_float4(ma[0], ma[1], ma[2], ma[3]);
                *reinterpret_cast<float4 *>(m1) = make_float4(mb[0], mb[1], mb[2], mb[3]);
                *reinterpret_cast<float4 *>(m2) = make_float4(mc[0], mc[1], mc[2], mc[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (gx + j < W) {
                        m0[j] = ma[j];
                        m1[j] = mb[j];
                        m2[j] = mc[j];
                    }
            }
        }
    }
    block_sum(s_acc, red, &part[tile].s);
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

__global__ __launch_bounds__(kThreads, 3) void k_ssim_grad(const float *__restrict__ x, const float *__restrict__ y,
                                                        int W, int H, Window win, const float *__restrict__ maps,
                                                        float w_l1, float w_ssim, float *__restrict__ dL_dc,
                                                        int aligned16, SsimPartial *__restrict__ part, int tiles_x,
                                                        int tiles)
{
    // one channel of the three coefficient maps on the tile + halo, and their column sums
    __shared__ float sin[3][kRH][kRWP];
    __shared__ __align__(16) float sv[3][kTH][kVW];
    __shared__ double red[kThreads / 64];
    const int t = threadIdx.x;
    const int tile = xcd_tile(tiles);
    const int x0 = (tile % tiles_x) * kTW, y0 = (tile / tiles_x) * kTH;
    const size_t plane = (size_t)W * H;
    const int hr = t / (kTW / 4), c4 = 4 * (t % (kTW / 4));
    const int gy = y0 + hr, gx = x0 + c4;
    // column pass: lane = column 0 .. 63 at rows vr0 .. vr0 + 3; lanes 0 .. 39 of each wave
    // also take one of the 160 outputs of columns 64 .. 73
    const int lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6), vr0 = kVR * wv;
    const int vb_e = kVB * wv + lane, vb_r = vb_e / kBW, vb_c = 64 + (vb_e - vb_r * kBW);
    const bool vb_in = lane < kVB;
    const bool row_ok = gy < H;
    const int nvalid = row_ok ? min(4, W - gx) : 0;   // this thread's pixels in the image
    const size_t o = ((size_t)gy * W + gx) * 3;
    const bool vec = aligned16 && nvalid == 4 && (o & 3) == 0;
    // x and y at the thread's four pixels, all channels (12 consecutive floats each)
    float xv[12], yv[12];
    if (vec) {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            *reinterpret_cast<float4 *>(&xv[4 * q]) = *reinterpret_cast<const float4 *>(x + o + 4 * q);
            *reinterpret_cast<float4 *>(&yv[4 * q]) = *reinterpret_cast<const float4 *>(y + o + 4 * q);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 12; ++k) {
            const bool in = k < 3 * nvalid;
            const size_t q = in ? o + k : 0;
            const float a = x[q], b = y[q];
            xv[k] = in ? a : 0.0f;
            yv[k] = in ? b : 0.0f;
        }
    }
    const StagePos P = stage_pos(W, H, x0, y0);
    Stage<3> st;
    {
        const char *const base[3] = {reinterpret_cast<const char *>(maps),
                                     reinterpret_cast<const char *>(maps + 3 * plane),
                                     reinterpret_cast<const char *>(maps + 6 * plane)};
        stage_load<3>(st, P, base, 4u);
    }
    stage_store<3>(st, sin);
    float g[12];
    double l1_acc = 0.0;
    for (int c = 0; c < 3; ++c) {
        __syncthreads();   // sin holds channel c; sv is free
        if (c < 2) {
            const size_t cp = (size_t)(c + 1) * plane;
            const char *const base[3] = {reinterpret_cast<const char *>(maps + cp),
                                         reinterpret_cast<const char *>(maps + 3 * plane + cp),
                                         reinterpret_cast<const char *>(maps + 6 * plane + cp)};
            stage_load<3>(st, P, base, 4u);
        }
        {   // columns 0 .. 63: lane = column, rows 4 w .. 4 w + 3 (14 input rows)
            float acc[3][kVR];
#pragma unroll
            for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int j = 0; j < kVR; ++j) acc[q][j] = 0.0f;
            float cv[3][kVR + 2 * kR];   // all reads issued before the first use
#pragma unroll
            for (int i = 0; i < kVR + 2 * kR; ++i)
#pragma unroll
                for (int q = 0; q < 3; ++q) cv[q][i] = sin[q][vr0 + i][lane];
#pragma unroll
            for (int i = 0; i < kVR + 2 * kR; ++i) {
                const float v[3] = {cv[0][i], cv[1][i], cv[2][i]};
#pragma unroll
                for (int j = 0; j < kVR; ++j)
                    if (i - j >= 0 && i - j < kTaps)
#pragma unroll
                        for (int q = 0; q < 3; ++q) acc[q][j] = fmaf(win.g[i - j], v[q], acc[q][j]);
            }
#pragma unroll
            for (int q = 0; q < 3; ++q)
#pragma unroll
                for (int j = 0; j < kVR; ++j) sv[q][vr0 + j][lane] = acc[q][j];
        }
        if (vb_in) {   // columns 64 .. 73: one output per lane
            float acc[3] = {0.0f, 0.0f, 0.0f};
            float cv[3][kTaps];
#pragma unroll
            for (int u = 0; u < kTaps; ++u)
#pragma unroll
                for (int q = 0; q < 3; ++q) cv[q][u] = sin[q][vb_r + u][vb_c];
#pragma unroll
            for (int u = 0; u < kTaps; ++u)
#pragma unroll
                for (int q = 0; q < 3; ++q) acc[q] = fmaf(win.g[u], cv[q][u], acc[q]);
#pragma unroll
            for (int q = 0; q < 3; ++q) sv[q][vb_r][vb_c] = acc[q];
        }
        __syncthreads();   // sv holds channel c; sin is free
        if (c < 2) stage_store<3>(st, sin);
        float rv[3][16];   // all reads issued before the first use
#pragma unroll
        for (int q = 0; q < 3; ++q) row_load14(&sv[q][hr][c4], rv[q]);
        float fa[4], fb[4], fc[4];
        row_filter4(rv[0], win, fa);
        row_filter4(rv[1], win, fb);
        row_filter4(rv[2], win, fc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float xq = xv[3 * j + c], yq = yv[3 * j + c];
            const float d = xq - yq;
            const float sg = d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f);
            l1_acc += (double)fabsf(d);   // zero outside the image
            const float gs = fmaf(2.0f * xq, fb[j], fmaf(yq, fc[j], fa[j]));   // N dSSIM/dx
            g[3 * j + c] = fmaf(w_l1, sg, -w_ssim * gs);
        }
    }
    if (vec) {
#pragma unroll
        for (int q = 0; q < 3; ++q) *reinterpret_cast<float4 *>(dL_dc + o + 4 * q) = *reinterpret_cast<float4 *>(&g[4 * q]);
    } else {
#pragma unroll
        for (int k = 0; k < 12; ++k)
            if (k < 3 * nvalid) dL_dc[o + k] = g[k];
    }
    block_sum(l1_acc, red, &part[tile].l1);
}

// The kernels' byte offsets (12 B per pixel of an image) fit in 32 bits.
bool index32(int32_t W, int32_t H) { return (uint64_t)W * (uint64_t)H * 12u < (uint64_t(1) << 32); }

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
    if (!index32(width, height)) return 0;
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
    if (!index32(width, height))
        return fail(GS_ERR_UNSUPPORTED, "image of %d x %d pixels: 12 W H must stay below 2^32", width, height);
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
    const int tiles = ws.gx * ws.gy;
    k_ssim_maps<<<(unsigned)tiles, kThreads, 0, stream>>>(color, target, width, height, win, maps, part, ws.gx, tiles);
    GS_LAUNCH_CHECK("k_ssim_maps");
    const double n = 3.0 * (double)width * (double)height;
    k_ssim_grad<<<(unsigned)tiles, kThreads, 0, stream>>>(color, target, width, height, win, maps,
                                               (float)((1.0 - (double)lambda) / n), (float)(0.5 * (double)lambda / n),
                                               dL_dcolor, (int)(aligned(color, 16) && aligned(target, 16) &&
                                                                aligned(dL_dcolor, 16)),
                                               part, ws.gx, tiles);
    GS_LAUNCH_CHECK("k_ssim_grad");
    k_ssim_final<<<1, kThreads, 0, stream>>>(part, ws.gx * ws.gy, 1.0 / n, (double)lambda, loss_out, ssim_out);
    GS_LAUNCH_CHECK("k_ssim_final");
    return GS_OK;
}
