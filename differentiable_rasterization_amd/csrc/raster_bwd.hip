// Backward rasterization (ByteSplat, section 2.1, Eq. 3 and Eq. 4).  Each pixel walks
// the entries it traversed in the forward pass back to front, recovering
// T_i = T_{i+1} / (1 - alpha_i) from the final transmittance, and forms the partial
// gradient of its loss with respect to the entry's screen-space fields:
//   dL/dc_i     = T_i alpha_i G
//   dL/dalpha_i = T_i (c_i - B_i) . G - G_T T_final / (1 - alpha_i),
//                 B_i = colour composited behind i (B = 0 after the last entry,
//                 B_{i-1} = alpha_i c_i + (1 - alpha_i) B_i)
//   unclamped alpha only: dL/do = dL/dalpha alpha / o, dL/dpower = dL/dalpha alpha,
//   dA = -dx^2/2 dpower, dB = -dx dy dpower, dC = -dy^2/2 dpower,
//   du = (A dx + B dy) dpower, dv = (B dx + C dy) dpower.
// Aggregation over pixels (Eq. 4): the four pixels of a lane share dx, so their
// contributions are first folded in registers, then summed over the wave with DPP
// (skipped when no lane of the wave touched the entry), and one lane per tile adds
// the tile's total for each entry to global memory with float atomics.
#include "kernels.h"
#include "raster.h"

namespace {

using namespace gsr;

template <bool HAS_GT>
__global__ __launch_bounds__(64) void k_raster_bwd(const int32_t *__restrict__ ranges, const uint32_t *__restrict__ ids,
                                                   const float2 *__restrict__ means2d,
                                                   const float4 *__restrict__ conic_o, const float *__restrict__ color,
                                                   int W, int H, int TX, int T, int per_xcd, float alpha_min,
                                                   float alpha_max, const float *__restrict__ t_final,
                                                   const int32_t *__restrict__ n_trav,
                                                   const float *__restrict__ dL_dc, const float *__restrict__ dL_dt,
                                                   float *__restrict__ grads2d, int64_t n)
{
    __shared__ float4 s0[kBatch], s1[kBatch], s2[kBatch], s3[kBatch];
    __shared__ float sacc[9][kBatch];
    __shared__ int sflag[kBatch];
    __shared__ uint32_t sid[kBatch];
    const int tile = (blockIdx.x % gsi::kXcds) * per_xcd + blockIdx.x / gsi::kXcds;
    if (tile >= T) return;
    const int lane = threadIdx.x;
    const int px = (tile % TX) * GS_TILE + (lane & 15);
    const int py0 = (tile / TX) * GS_TILE + (lane >> 4) * kPix;
    const float fx = (float)px + 0.5f;
    float fy[kPix], Tr[kPix], Tf[kPix], G0[kPix], G1[kPix], G2[kPix], GT[kPix], B0[kPix], B1[kPix], B2[kPix];
    int np[kPix];
    int nmax = 0;
#pragma unroll
    for (int k = 0; k < kPix; ++k) {
        const int py = py0 + k;
        fy[k] = (float)py + 0.5f;
        B0[k] = B1[k] = B2[k] = 0.0f;
        if (px < W && py < H) {
            const size_t idx = (size_t)py * W + px;
            Tr[k] = Tf[k] = t_final[idx];
            np[k] = n_trav[idx];
            G0[k] = dL_dc[3 * idx];
            G1[k] = dL_dc[3 * idx + 1];
            G2[k] = dL_dc[3 * idx + 2];
            GT[k] = HAS_GT ? dL_dt[idx] : 0.0f;
        } else {
            Tr[k] = Tf[k] = 1.0f;
            np[k] = 0;
            G0[k] = G1[k] = G2[k] = GT[k] = 0.0f;
        }
        nmax = max(nmax, np[k]);
    }
    nmax = gsd::wave_max_i32(nmax);
    const int start = ranges[tile];
    nmax = min(nmax, ranges[tile + 1] - start);   // n_trav never exceeds the list; guard against misuse
    for (int bend = start + nmax; bend > start; bend -= kBatch) {
        const int b0 = max(start, bend - kBatch);
        const int cnt = bend - b0;
        if (lane < cnt) {
            const uint32_t gid = ids[b0 + lane];
            const Entry en = make_entry(gid, means2d, conic_o, color);
            sid[lane] = gid;
            s0[lane] = en.p0;
            s1[lane] = en.p1;
            s2[lane] = en.p2;
            s3[lane] = en.p3;
        }
        __syncthreads();
        for (int j = cnt - 1; j >= 0; --j) {
            const int rel = b0 + j - start;
            const float4 p0 = s0[j], p1 = s1[j], p2 = s2[j];
            const float inv_o = s3[j].x;
            const float dx = fx - p0.x;
            const float base = fmaf(p0.z * dx, dx, p1.y);
            const float bdx = p0.w * dx;
            float sum0 = 0.0f, sum1 = 0.0f, sum2 = 0.0f, s_o = 0.0f, s_r = 0.0f, s_g = 0.0f, s_b = 0.0f;
            bool touched = false;
#pragma unroll
            for (int k = 0; k < kPix; ++k) {
                const float dy = fy[k] - p0.y;
                const float raw = exp2_fast(exponent(base, bdx, p1.x, dy));
                const float alpha = fminf(alpha_max, raw);
                if (rel < np[k] && alpha >= alpha_min) {
                    const float om = 1.0f - alpha;
                    const float Ti = Tr[k] * __builtin_amdgcn_rcpf(om);
                    const float w = Ti * alpha;
                    s_r = fmaf(w, G0[k], s_r);
                    s_g = fmaf(w, G1[k], s_g);
                    s_b = fmaf(w, G2[k], s_b);
                    float dal = Ti * ((p1.z - B0[k]) * G0[k] + (p1.w - B1[k]) * G1[k] + (p2.x - B2[k]) * G2[k]);
                    if (HAS_GT) dal -= GT[k] * Tf[k] * __builtin_amdgcn_rcpf(om);
                    if (raw < alpha_max) {
                        const float dpow = dal * alpha;
                        s_o = fmaf(dpow, inv_o, s_o);
                        sum0 += dpow;
                        sum1 = fmaf(dy, dpow, sum1);
                        sum2 = fmaf(dy * dy, dpow, sum2);
                    }
                    B0[k] = fmaf(alpha, p1.z - B0[k], B0[k]);
                    B1[k] = fmaf(alpha, p1.w - B1[k], B1[k]);
                    B2[k] = fmaf(alpha, p2.x - B2[k], B2[k]);
                    Tr[k] = Ti;
                    touched = true;
                }
            }
            if (__ballot(touched) == 0) {
                if (lane == 63) sflag[j] = 0;
                continue;
            }
            // fold the four pixels into the 9 fields: (u, v, A, B, C, o, r, g, b)
            const float A = p2.y, Bc = p2.z, C = p2.w;
            float f[9];
            f[0] = fmaf(A * dx, sum0, Bc * sum1);
            f[1] = fmaf(Bc * dx, sum0, C * sum1);
            f[2] = -0.5f * dx * dx * sum0;
            f[3] = -dx * sum1;
            f[4] = -0.5f * sum2;
            f[5] = s_o;
            f[6] = s_r;
            f[7] = s_g;
            f[8] = s_b;
#pragma unroll
            for (int q = 0; q < 9; ++q) f[q] = gsd::wave_sum_to_lane63(f[q]);
            if (lane == 63) {
#pragma unroll
                for (int q = 0; q < 9; ++q) sacc[q][j] = f[q];
                sflag[j] = 1;
            }
        }
        __syncthreads();
        if (lane < cnt && sflag[lane]) {
            const uint32_t g = sid[lane];
#pragma unroll
            for (int q = 0; q < 9; ++q) {
                const float v = sacc[q][lane];
                if (v != 0.0f) atomicAdd(grads2d + (size_t)q * n + g, v);
            }
        }
        __syncthreads();
    }
}

}  // namespace

namespace gsi {
gs_status check_raster_inputs(const gs_projected *proj, const gs_bins *bins);
}

extern "C" gs_status gs_raster_bwd(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                                   const gs_camera *cam, const gs_raster_params *p, const float *t_final,
                                   const int32_t *n_trav, const float *dL_dcolor, const float *dL_dt, float *grads2d,
                                   gs_param_grads *grads3d, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(proj, bins)) != GS_OK) return s;
    if (!t_final || !n_trav || !dL_dcolor || (g->n > 0 && !grads2d))
        return fail(GS_ERR_INVALID_ARGUMENT, "t_final / n_trav / dL_dcolor / grads2d is NULL");
    if (bins->capacity > 0 && !bins->ids) return fail(GS_ERR_INVALID_ARGUMENT, "ids is NULL");
    const int64_t n = g->n;
    if ((s = fill_f32(grads2d, 9 * n, 0.0f, stream)) != GS_OK) return s;
    const int TX = tiles_x(cam->width), T = TX * tiles_y(cam->height);
    const int per = xcd_per(T);
    const dim3 grid((unsigned)(per * kXcds)), block(64);
    const float2 *m2 = reinterpret_cast<const float2 *>(proj->means2d);
    const float4 *co = reinterpret_cast<const float4 *>(proj->conic_opacity);
    if (n > 0) {
        if (dL_dt)
            k_raster_bwd<true><<<grid, block, 0, stream>>>(bins->tile_ranges, bins->ids, m2, co, proj->color,
                                                           cam->width, cam->height, TX, T, per, p->alpha_min,
                                                           p->alpha_max, t_final, n_trav, dL_dcolor, dL_dt, grads2d, n);
        else
            k_raster_bwd<false><<<grid, block, 0, stream>>>(bins->tile_ranges, bins->ids, m2, co, proj->color,
                                                            cam->width, cam->height, TX, T, per, p->alpha_min,
                                                            p->alpha_max, t_final, n_trav, dL_dcolor, nullptr,
                                                            grads2d, n);
        GS_LAUNCH_CHECK("k_raster_bwd");
    }
    if (grads3d) return launch_project_bwd(g, cam, p, grads2d, grads3d, stream);
    return GS_OK;
}
