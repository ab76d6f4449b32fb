// Forward rasterization: front-to-back alpha compositing per 16x16 tile
// (ByteSplat, section 2.1, Eq. 1): C(p) = sum_i T_i alpha_i c_i,
// T_i = prod_{j<i} (1 - alpha_j), with the alpha-check (alpha < alpha_min skips the
// entry) and termination once T_i < theta_T.
#include "raster.h"

namespace {

using namespace gsr;

__global__ __launch_bounds__(64) void k_raster_fwd(const int32_t *__restrict__ ranges, const uint32_t *__restrict__ ids,
                                                   const float2 *__restrict__ means2d,
                                                   const float4 *__restrict__ conic_o, const float *__restrict__ color,
                                                   int W, int H, int TX, int T, int per_xcd, float alpha_min,
                                                   float alpha_max, float t_min, float *__restrict__ out_c,
                                                   float *__restrict__ out_t, int32_t *__restrict__ out_n,
                                                   unsigned long long *__restrict__ n_sum)
{
    __shared__ float4 s0[kBatch], s1[kBatch], s2[kBatch];
    const int tile = (blockIdx.x % gsi::kXcds) * per_xcd + blockIdx.x / gsi::kXcds;
    if (tile >= T) return;
    const int lane = threadIdx.x;
    const int px = (tile % TX) * GS_TILE + (lane & 15);
    const int py0 = (tile / TX) * GS_TILE + (lane >> 4) * kPix;
    const float fx = (float)px + 0.5f;
    float fy[kPix], Tr[kPix], cr[kPix], cg[kPix], cb[kPix];
    int nt[kPix];
    bool live[kPix];
#pragma unroll
    for (int k = 0; k < kPix; ++k) {
        fy[k] = (float)(py0 + k) + 0.5f;
        Tr[k] = 1.0f;
        cr[k] = cg[k] = cb[k] = 0.0f;
        nt[k] = -1;
        live[k] = px < W && py0 + k < H;
    }
    const int start = ranges[tile], end = ranges[tile + 1];
    for (int b0 = start; b0 < end; b0 += kBatch) {
        const bool any = live[0] | live[1] | live[2] | live[3];
        if (__ballot(any) == 0) break;
        const int e = b0 + lane;
        if (e < end) {
            const Entry en = make_entry(ids[e], means2d, conic_o, color);
            s0[lane] = en.p0;
            s1[lane] = en.p1;
            s2[lane] = en.p2;
        }
        __syncthreads();
        const int cnt = min(kBatch, end - b0);
        for (int j = 0; j < cnt; ++j) {
            const float4 p0 = s0[j], p1 = s1[j];
            const float blue = s2[j].x;
            const float dx = fx - p0.x;
            const float base = fmaf(p0.z * dx, dx, p1.y);
            const float bdx = p0.w * dx;
#pragma unroll
            for (int k = 0; k < kPix; ++k) {
                const float dy = fy[k] - p0.y;
                const float alpha = fminf(alpha_max, exp2_fast(exponent(base, bdx, p1.x, dy)));
                if (live[k] && alpha >= alpha_min) {
                    const float w = Tr[k] * alpha;
                    cr[k] = fmaf(w, p1.z, cr[k]);
                    cg[k] = fmaf(w, p1.w, cg[k]);
                    cb[k] = fmaf(w, blue, cb[k]);
                    Tr[k] = Tr[k] * (1.0f - alpha);
                    if (Tr[k] < t_min) {
                        live[k] = false;
                        nt[k] = b0 + j + 1 - start;
                    }
                }
            }
        }
        __syncthreads();
    }
    int lane_sum = 0;
#pragma unroll
    for (int k = 0; k < kPix; ++k) {
        const int py = py0 + k;
        if (px < W && py < H) {
            const size_t idx = (size_t)py * W + px;
            const int np = nt[k] >= 0 ? nt[k] : end - start;
            out_c[3 * idx] = cr[k];
            out_c[3 * idx + 1] = cg[k];
            out_c[3 * idx + 2] = cb[k];
            out_t[idx] = Tr[k];
            out_n[idx] = np;
            lane_sum += np;
        }
    }
    if (n_sum) {
        const unsigned tot = gsd::wave_sum_u32_to_lane63((unsigned)lane_sum);
        if (lane == 63 && tot > 0u) atomicAdd(n_sum, (unsigned long long)tot);
    }
}

}  // namespace

namespace gsi {

gs_status check_raster_inputs(const gs_projected *proj, const gs_bins *bins)
{
    if (!proj || !bins) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!bins->tile_ranges) return fail(GS_ERR_INVALID_ARGUMENT, "tile_ranges is NULL");
    if (!proj->means2d || !proj->conic_opacity || !proj->color)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected means2d / conic_opacity / color is NULL");
    if (!aligned(proj->conic_opacity, 16) || !aligned(proj->means2d, 8))
        return fail(GS_ERR_INVALID_ARGUMENT, "conic_opacity must be 16-byte, means2d 8-byte aligned");
    return GS_OK;
}

}  // namespace gsi

extern "C" gs_status gs_raster_fwd(const gs_projected *proj, const gs_bins *bins, const gs_camera *cam,
                                   const gs_raster_params *p, float *color, float *t_final, int32_t *n_trav,
                                   unsigned long long *n_trav_sum, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(proj, bins)) != GS_OK) return s;
    if (!color || !t_final || !n_trav) return fail(GS_ERR_INVALID_ARGUMENT, "an output pointer is NULL");
    if (bins->capacity > 0 && !bins->ids) return fail(GS_ERR_INVALID_ARGUMENT, "ids is NULL");
    const int TX = tiles_x(cam->width), T = TX * tiles_y(cam->height);
    const int per = xcd_per(T);
    k_raster_fwd<<<(unsigned)(per * kXcds), 64, 0, stream>>>(
        bins->tile_ranges, bins->ids, reinterpret_cast<const float2 *>(proj->means2d),
        reinterpret_cast<const float4 *>(proj->conic_opacity), proj->color, cam->width, cam->height, TX, T, per,
        p->alpha_min, p->alpha_max, p->t_min, color, t_final, n_trav, n_trav_sum);
    GS_LAUNCH_CHECK("k_raster_fwd");
    return GS_OK;
}
