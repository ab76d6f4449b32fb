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
#include "raster.h"

namespace {

using namespace gsr;

constexpr int kBwdBatch = 4;   // entries per transpose-reduction (4 x 9 values -> 4 rows of 16 lanes)
constexpr int kFields = 9;

__device__ __forceinline__ float swap_add32(float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap_add16(float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v[e * 9 + f] holds this lane's value of field f of entry e (e < 4).  Sums every field
// of every entry over the 64 lanes, transposing as it goes so that each sum lands in one
// lane: afterwards lane (e, n) of row e = lane >> 4 (n = lane & 15) holds the total of
// field F(n) = 4 b1 + 2 b2 + b3 of entry e (b_k = bit k of n; lanes n and n ^ 1 hold the
// same field) and t8 holds the total of field 8 of entry e.
//   1. v_permlane32_swap + add: rows 0-1 keep entries 0-1, rows 2-3 entries 2-3
//   2. v_permlane16_swap + add: row e keeps entry e (9 partial sums per lane)
//   3. within each 16-lane row, fields 0-7 by a transposing butterfly (partners n ^ 8 by
//      row_ror:8, n ^ 7 by row_half_mirror, n ^ 2 and n ^ 1 by quad_perm): at each step a
//      lane keeps one field of each pair, chosen by one bit of n, adds the partner's value
//      of that field, and passes on the other; field 8 by a plain butterfly.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    using namespace gsd;
    // old = 0 (the identity of +) lets the compiler fold the move into the DPP add
    return f_from_i(__builtin_amdgcn_update_dpp(0, i_from_f(v), CTRL, 0xF, 0xF, false));
}

constexpr int kRowRor8 = 0x128;

// One transposing step: keep x if !bit else y, and add the partner's copy of the same field.
template <int CTRL>
__device__ __forceinline__ float tstep(float x, float y, bool bit)
{
    const float keep = bit ? y : x, send = bit ? x : y;
    return keep + dpp_f<CTRL>(send);
}

// Per-lane choice of one of four wave-uniform values by the lane's row (lane >> 4).
__device__ __forceinline__ float by_row(int row, float a0, float a1, float a2, float a3)
{
    const float lo = (row & 1) ? a1 : a0, hi = (row & 1) ? a3 : a2;
    return (row & 2) ? hi : lo;
}

__device__ __forceinline__ void reduce_4x9(float (&v)[kBwdBatch * kFields], int n, float &fz, float &t8)
{
    using namespace gsd;
#pragma unroll
    for (int i = 0; i < 18; ++i) v[i] = swap_add32(v[i], v[i + 18]);   // lanes < 32: slot i, else slot i + 18
#pragma unroll
    for (int i = 0; i < 9; ++i) v[i] = swap_add16(v[i], v[i + 9]);     // row r: slot i + 9 r
    const bool b3 = (n >> 3) & 1, b2 = (n >> 2) & 1, b1 = (n >> 1) & 1;
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = tstep<kRowRor8>(v[2 * k], v[2 * k + 1], b3);   // field 2k + b3
    const float x0 = tstep<kRowHalfMirror>(w[0], w[1], b2);                            // field 2 b2 + b3
    const float x1 = tstep<kRowHalfMirror>(w[2], w[3], b2);                            // 4 + 2 b2 + b3
    const float y = tstep<kQuadSwap2>(x0, x1, b1);                                     // 4 b1 + 2 b2 + b3
    fz = y + dpp_f<kQuadSwap1>(y);
    float z = v[8];
    z += dpp_f<kQuadSwap1>(z);
    z += dpp_f<kQuadSwap2>(z);
    z += dpp_f<kRowHalfMirror>(z);
    z += dpp_f<kRowRor8>(z);
    t8 = z;
}

template <bool HAS_GT>
__global__ __launch_bounds__(64) void k_raster_bwd(const int32_t *__restrict__ ranges, const int32_t *__restrict__ order,
                                                   const float4 *__restrict__ qrec, const uint64_t *__restrict__ bitmap,
                                                   const uint32_t *__restrict__ wpre, int64_t words, int W, int H,
                                                   int TX, int T, float alpha_min, float alpha_max,
                                                   const float *__restrict__ color, const float *__restrict__ t_final,
                                                   const int32_t *__restrict__ n_trav, const float *__restrict__ dL_dc,
                                                   const float *__restrict__ dL_dt,
                                                   const BinsHeader *__restrict__ hdr, float *__restrict__ qgrad,
                                                   uint32_t *__restrict__ qstamp)
{
    int tidx, q;
    raster_block(tidx, q);
    if (tidx >= T) return;
    const int tile = order[tidx];
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
    const uint32_t epoch = hdr->epoch;
    const int row = lane >> 4, nl = lane & 15;
    // the reduced field each lane of a row holds (reduce_4x9): even lanes hold fields 0-7,
    // lane 1 field 8; lane 3 writes the slot's stamp (epoch, ~epoch)
    const bool stamp_lane = nl == 3;
    const int my_field = nl == 1 ? 8 : 4 * ((nl >> 1) & 1) + 2 * ((nl >> 2) & 1) + ((nl >> 3) & 1);
    const bool lane_writes = (nl & 1) == 0 || nl == 1 || stamp_lane;
    const uint2 stamp = make_uint2(epoch, ~epoch);
    float Tr = 1.0f;
    // L2 prefetch of the next chunk of 64 records ahead of the scalar reads
    uint32_t sink = prefetch_records(qrec, j0, j1), pend = prefetch_records(qrec, j0 + 64u, j1);
    for (uint32_t jt = j0; jt < j1;) {
        if (((jt - j0) & 63u) == 0u && jt > j0) {
            sink ^= pend;
            pend = prefetch_records(qrec, jt + 64u, j1);
        }
        // records jt .. jt+3 (past j1: spare, unused); one wait per batch
        float4 p0[kBwdBatch], p1[kBwdBatch];
        float blue[kBwdBatch], kent[kBwdBatch], slot[kBwdBatch];
        const float4 *rb = qrec + kRecF4 * (size_t)jt;
#pragma unroll
        for (int i = 0; i < kBwdBatch; ++i) {
            p0[i] = rb[kRecF4 * i];
            p1[i] = rb[kRecF4 * i + 1];
            const float4 p2 = rb[kRecF4 * i + 2];
            blue[i] = p2.x;
            kent[i] = p2.z;
            slot[i] = p2.w;
        }
#pragma unroll
        for (int i = 0; i < kBwdBatch; ++i)
            asm volatile("" ::"s"(p0[i].x), "s"(p0[i].y), "s"(p0[i].z), "s"(p0[i].w), "s"(p1[i].x), "s"(p1[i].y),
                         "s"(p1[i].z), "s"(p1[i].w), "s"(blue[i]), "s"(kent[i]), "s"(slot[i]));
        const uint32_t cnt = min((uint32_t)kBwdBatch, j1 - jt);
        float v[kBwdBatch * kFields];
        bool any = false;
#pragma unroll
        for (int i = 0; i < kBwdBatch; ++i) {
            float *o = v + kFields * i;
            const int rel = (int)__float_as_uint(kent[i]) - start;
            const float dx = fx - p0[i].x, dy = fy - p0[i].y;
            const float raw = exp2_fast(exponent(p0[i], p1[i], dx, dy));
            // the forward pass's alpha and T, bit for bit
            const float alpha = fminf(alpha_max, raw);
            const bool take = (uint32_t)i < cnt && rel < np && alpha >= alpha_min;
            const float a = take ? alpha : 0.0f;
            const float om = 1.0f - a;
            const float ro = __builtin_amdgcn_rcpf(om);
            const float w = Tr * a;
            o[6] = w * G0;
            o[7] = w * G1;
            o[8] = w * G2;
            const float cg = fmaf(p1[i].z, G0, fmaf(p1[i].w, G1, blue[i] * G2));
            Z = fmaf(-w, cg, Z);
            const float dal = fmaf(Tr, cg, -ro * Z);
            const float s0 = dal * (raw < alpha_max ? a : 0.0f);   // clamped alpha has no power gradient
            o[0] = s0;
            o[1] = dx * s0;
            o[2] = dy * s0;
            o[3] = dx * o[1];
            o[4] = dy * o[1];
            o[5] = dy * o[2];
            Tr = Tr * om;
            any |= take;
        }
        // gradient slot of the batch's record e = row (record jt + e); lane n writes field
        // my_field (see reduce_4x9)
        const uint32_t my_slot = __float_as_uint(by_row(row, slot[0], slot[1], slot[2], slot[3]));
        float *dst = qgrad + (size_t)my_slot * kGradSlot + my_field;
        uint2 *dst_stamp = reinterpret_cast<uint2 *>(qstamp) + my_slot;
        const bool writer = (uint32_t)row < cnt && lane_writes;
        jt += cnt;
        if (__ballot(any) == 0) continue;   // no pixel takes these records: slots left unstamped
        float fz, t8;
        reduce_4x9(v, nl, fz, t8);
        if (writer) {
            if (stamp_lane)
                *dst_stamp = stamp;
            else
                *dst = nl == 1 ? t8 : fz;
        }
    }
    sink ^= pend;
    asm volatile("" ::"v"(sink));
}

// A new stamp for the gradient slots of this backward call.
__global__ void k_new_epoch(BinsHeader *__restrict__ hdr) { hdr->epoch = hdr->epoch + 1u; }

// Eq. 4: the gradient of Gaussian g is the sum of the slots of its quadrant records,
// slots qoff[g] .. qoff[g + 1], added in order.  Every Gaussian is
// written, culled ones (no records) with zeros, and all of them when the lists did not
// fit the capacity.  One thread per Gaussian, in index order
// so that the stores coalesce.
__global__ __launch_bounds__(256) void k_grad_reduce(const BinsHeader *__restrict__ hdr,
                                                     const uint32_t *__restrict__ qoff, const float4 *__restrict__ qgrad,
                                                     const uint2 *__restrict__ qstamp,
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
    const float4 *rc = reinterpret_cast<const float4 *>(rb + L.qrec) + kRecPad * kRecF4;
    const uint64_t *bm = reinterpret_cast<const uint64_t *>(rb + L.bitmap);
    const uint32_t *wp = reinterpret_cast<const uint32_t *>(rb + L.wpre);
    float *qg = reinterpret_cast<float *>(rb + L.qgrad);
    uint32_t *qs = reinterpret_cast<uint32_t *>(rb + L.qstamp);
    const unsigned grid = (unsigned)raster_grid(T);
    BinsHeader *hdr = reinterpret_cast<BinsHeader *>(rb + L.hdr);
    k_new_epoch<<<1, 1, 0, stream>>>(hdr);
    GS_LAUNCH_CHECK("k_new_epoch");
    if (dL_dt)
        k_raster_bwd<true><<<grid, 64, 0, stream>>>(bins->tile_ranges, order, rc, bm, wp, L.words, cam->width,
                                                    cam->height, TX, T, p->alpha_min, p->alpha_max, color, t_final,
                                                    n_trav, dL_dcolor, dL_dt, hdr, qg, qs);
    else
        k_raster_bwd<false><<<grid, 64, 0, stream>>>(bins->tile_ranges, order, rc, bm, wp, L.words, cam->width,
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
            reinterpret_cast<const float4 *>(rb + L.qgrad), reinterpret_cast<const uint2 *>(rb + L.qstamp),
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
