// Backward rasterization (ByteSplat, section 2.1, Eq. 3 and Eq. 4).  Each pixel walks
// the entries it traversed in the forward pass front to back, recomputing T_i exactly as
// the forward pass did (T_1 = 1, T_{i+1} = T_i (1 - alpha_i)), and forms the partial
// gradient of its loss with respect to the entry's screen-space fields:
//   dL/dc_i     = T_i alpha_i G
//   dL/dalpha_i = T_i c_i . G - (T_i B_i . G + G_T T_final) / (1 - alpha_i)
//                 with T_i B_i = sum_{j>i} T_j alpha_j c_j / (1 - alpha_i) the colour
//                 composited behind i, so T_i B_i . G (1 - alpha_i) = C . G - sum_{j<=i}
//                 T_j alpha_j c_j . G, C the pixel's final colour from the forward pass
//   unclamped alpha only: dL/dpower = dL/dalpha alpha, dL/do = dL/dpower / o,
//   dA = -dx^2/2 dpower, dB = -dx dy dpower, dC = -dy^2/2 dpower,
//   du = (A dx + B dy) dpower, dv = (B dx + C dy) dpower.
// Walking front to back keeps T_i exact where T_final underflows (theta_T = 0 with deep
// lists), which the back-to-front recovery T_i = T_{i+1} / (1 - alpha_i) cannot.
// Aggregation over pixels (Eq. 4), without atomics: each lane forms the per-pixel moments
//   S0 = dpower, Sx = dx S0, Sy = dy S0, Sxx = dx Sx, Sxy = dy Sx, Syy = dy Sy and the
//   colour terms T_i alpha_i G for 4 records at a time; the wave sums the 36 values in one
//   transposing reduction (reduce_4x9), after which 9 lanes of row e hold the 9 totals of
//   record e, and stores them in the record's gradient slot (one store instruction for
//   the 36 values).  The screen-space gradients are linear in these sums with coefficients
//   of the Gaussian alone,
//     du = A Sx + B Sy, dv = B Sx + C Sy, dA = -Sxx/2, dB = -Sxy, dC = -Syy/2, do = S0 / o,
//   so they are formed once per Gaussian, after its slots are summed (sum_slots in
//   raster.h).  The binning gives each Gaussian's quadrant records consecutive slots: the
//   sum of Eq. 4 is one contiguous run of slots added in a fixed order, so the gradients
//   are deterministic.
//
// Lanes that do not take an entry run the same instructions with alpha = 0, which leaves
// T unchanged and contributes zeros (no divergent branches).
//
// One wave per 8x8 quadrant (see raster.h), walking its tile's record list for the
// quadrant front to back up to the furthest entry any of its pixels traversed.  The slots of
// records behind that point, and of batches no pixel takes, are not written: every slot
// written carries the call's stamp (BinsHeader::epoch), and the per-Gaussian sums skip the
// others.
#include "kernels.h"
#include "raster_walk.h"

namespace {

using namespace gsr;

constexpr int kFields = 9;

template <bool HAS_GT>
__global__ __launch_bounds__(64) void k_raster_bwd(const int32_t *__restrict__ ranges, const int32_t *__restrict__ order,
                                                   const uint2 *__restrict__ qent, const float4 *__restrict__ grec,
                                                   const uint64_t *__restrict__ bitmap,
                                                   const uint32_t *__restrict__ wpre, int64_t words, int W, int H,
                                                   int TX, int T, float alpha_min, float alpha_max,
                                                   const float *__restrict__ color, const float *__restrict__ t_final,
                                                   const int32_t *__restrict__ n_trav, const float *__restrict__ dL_dc,
                                                   const float *__restrict__ dL_dt,
                                                   const BinsHeader *__restrict__ hdr, float *__restrict__ qgrad,
                                                   uint32_t *__restrict__ qstamp)
{
    int tile, q;
    raster_block(order, tile, q);
    const int lane = threadIdx.x;
    const int px = (tile % TX) * GS_TILE + (q & 1) * 8 + (lane & 7);
    const int py = (tile / TX) * GS_TILE + (q >> 1) * 8 + (lane >> 3);
    const bool inside = px < W && py < H;
    const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
    // Z = C . G + G_T T_final - sum_{j<=i} T_j alpha_j c_j . G  =  (T_i B_i . G + G_T T_final) (1 - alpha_i)
    float G0 = 0.0f, G1 = 0.0f, G2 = 0.0f, Z = 0.0f;
    int np = 0;
    if (inside) {
        const size_t idx = (size_t)py * W + px;
        np = n_trav[idx];
        G0 = dL_dc[3 * idx];
        G1 = dL_dc[3 * idx + 1];
        G2 = dL_dc[3 * idx + 2];
        Z = fmaf(color[3 * idx], G0, fmaf(color[3 * idx + 1], G1, color[3 * idx + 2] * G2));
        if (HAS_GT) Z = fmaf(dL_dt[idx], t_final[idx], Z);
    }
    const int start = ranges[tile], end = ranges[tile + 1];
    if (start >= end) return;   // empty list: no records, no slots (the prefix counts may be unset)
    // the wave walks up to the furthest entry any of its pixels traversed
    const int nmax = max(0, min(gsd::wave_max_i32(np), end - start));
    const uint64_t *bq = bitmap + (int64_t)q * words;
    const uint32_t *wq = wpre + (int64_t)q * (words + 1);
    const uint32_t j0 = quad_prefix(bq, wq, (uint32_t)start), j1 = quad_prefix(bq, wq, (uint32_t)(start + nmax));
    // this pixel's records: those before the first entry beyond its N_p
    const uint32_t jend = quad_prefix(bq, wq, (uint32_t)(start + max(0, min(np, end - start))));
    bwd_walk(qent, grec, j0, j1, fx, fy, jend, G0, G1, G2, Z, alpha_min, alpha_max, hdr->epoch, qgrad, qstamp);
}

// A new stamp for the gradient slots of this backward call.
__global__ void k_new_epoch(BinsHeader *__restrict__ hdr) { hdr->epoch = next_epoch(hdr->epoch); }

// Eq. 4: the gradient of Gaussian g is the sum of the slots of its quadrant records,
// slots qoff[g] .. qoff[g + 1], added in order.  Every Gaussian is
// written, culled ones (no records) with zeros, and all of them when the lists did not
// fit the capacity.  One thread per Gaussian, in index order
// so that the stores coalesce.
__global__ __launch_bounds__(256) void k_grad_reduce(const BinsHeader *__restrict__ hdr,
                                                     const uint32_t *__restrict__ qoff, const float4 *__restrict__ qgrad,
                                                     const uint32_t *__restrict__ qstamp,
                                                     const float4 *__restrict__ rec, int64_t n,
                                                     float *__restrict__ grads2d)
{
    __shared__ SlotStage stage[4];
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float acc[kFields];
    sum_slots(hdr, qoff, qgrad, qstamp, rec, g, n, stage[threadIdx.x >> 6], acc);
    if (g >= n) return;
#pragma unroll
    for (int f = 0; f < kFields; ++f) grads2d[(size_t)f * n + g] = acc[f];
}

}  // namespace

namespace gsi {
gs_status check_raster_inputs(const gs_bins *bins, const gs_camera *cam);
}

extern "C" gs_status gs_raster_bwd_partials(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam,
                                            const gs_raster_params *p, const float *color, const float *t_final,
                                            const int32_t *n_trav, const float *dL_dcolor, const float *dL_dt,
                                            hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(bins, cam)) != GS_OK) return s;
    if (!color || !t_final || !n_trav || !dL_dcolor)
        return fail(GS_ERR_INVALID_ARGUMENT, "color / t_final / n_trav / dL_dcolor is NULL");
    const int64_t n = g->n;
    if (n == 0) return GS_OK;
    const int TX = tiles_x(cam->width), T = TX * tiles_y(cam->height);
    const RasterLayout L = raster_layout(n, bins->capacity, T);
    char *rb = static_cast<char *>(bins->raster);
    const int32_t *order = reinterpret_cast<const int32_t *>(rb + L.order);
    const uint2 *qe = reinterpret_cast<const uint2 *>(rb + L.qent);
    const float4 *gr = reinterpret_cast<const float4 *>(rb + L.grec);
    const uint64_t *bm = reinterpret_cast<const uint64_t *>(rb + L.bitmap);
    const uint32_t *wp = reinterpret_cast<const uint32_t *>(rb + L.wpre);
    float *qg = reinterpret_cast<float *>(rb + L.qgrad);
    uint32_t *qs = reinterpret_cast<uint32_t *>(rb + L.qstamp);
    const unsigned grid = (unsigned)raster_grid(T);
    BinsHeader *hdr = reinterpret_cast<BinsHeader *>(rb + L.hdr);
    k_new_epoch<<<1, 1, 0, stream>>>(hdr);
    GS_LAUNCH_CHECK("k_new_epoch");
    if (dL_dt)
        k_raster_bwd<true><<<grid, 64, 0, stream>>>(bins->tile_ranges, order, qe, gr, bm, wp, L.words, cam->width,
                                                    cam->height, TX, T, p->alpha_min, p->alpha_max, color, t_final,
                                                    n_trav, dL_dcolor, dL_dt, hdr, qg, qs);
    else
        k_raster_bwd<false><<<grid, 64, 0, stream>>>(bins->tile_ranges, order, qe, gr, bm, wp, L.words, cam->width,
                                                     cam->height, TX, T, p->alpha_min, p->alpha_max, color, t_final,
                                                     n_trav, dL_dcolor, nullptr, hdr, qg, qs);
    GS_LAUNCH_CHECK("k_raster_bwd");
    return GS_OK;
}

extern "C" gs_status gs_grad_aggregate(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                                       const gs_camera *cam, const gs_raster_params *p, float *grads2d,
                                       gs_param_grads *grads3d, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(bins, cam)) != GS_OK) return s;
    if (g->n > 0 && !grads2d) return fail(GS_ERR_INVALID_ARGUMENT, "grads2d is NULL");
    if (g->n > 0 && (!proj || !proj->rec || !aligned(proj->rec, 16)))
        return fail(GS_ERR_INVALID_ARGUMENT, "proj->rec is NULL or not 16-byte aligned");
    const int64_t n = g->n;
    if (n > 0) {
        const int T = tiles_x(cam->width) * tiles_y(cam->height);
        const RasterLayout L = raster_layout(n, bins->capacity, T);
        const char *rb = static_cast<const char *>(bins->raster);
        k_grad_reduce<<<(unsigned)ceil_div(n, 256), 256, 0, stream>>>(
            reinterpret_cast<const BinsHeader *>(rb + L.hdr), reinterpret_cast<const uint32_t *>(rb + L.qoff),
            reinterpret_cast<const float4 *>(rb + L.qgrad), reinterpret_cast<const uint32_t *>(rb + L.qstamp),
            reinterpret_cast<const float4 *>(proj->rec), n, grads2d);
        GS_LAUNCH_CHECK("k_grad_reduce");
    }
    if (grads3d) return launch_project_bwd(g, cam, p, grads2d, grads3d, stream);
    return GS_OK;
}

extern "C" gs_status gs_raster_bwd(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                                   const gs_camera *cam, const gs_raster_params *p, const float *color,
                                   const float *t_final, const int32_t *n_trav, const float *dL_dcolor,
                                   const float *dL_dt, float *grads2d, gs_param_grads *grads3d, hipStream_t stream)
{
    if (g && g->n > 0 && !grads2d) return gsi::fail(GS_ERR_INVALID_ARGUMENT, "grads2d is NULL");
    const gs_status s = gs_raster_bwd_partials(g, bins, cam, p, color, t_final, n_trav, dL_dcolor, dL_dt, stream);
    if (s != GS_OK) return s;
    return gs_grad_aggregate(g, proj, bins, cam, p, grads2d, grads3d, stream);
}
