// Forward rasterization: front-to-back alpha compositing per 16x16 tile
// (ByteSplat, section 2.1, Eq. 1): C(p) = sum_i T_i alpha_i c_i,
// T_i = prod_{j<i} (1 - alpha_j), with the alpha-check (alpha < alpha_min skips the
// entry) and termination once T_i < theta_T.
//
// One wave per 8x8 quadrant (see raster.h): the wave walks its tile's record list for the
// quadrant (the entries whose box reaches it, in list order) and stops as soon as every
// pixel of the quadrant has terminated.  N_p counts every entry of the 16x16 tile list up
// to the termination point (the Gaussians the pixel traverses), whether or not the
// quadrant's list holds them.
#include "raster_walk.h"

namespace {

using namespace gsr;

__global__ __launch_bounds__(64) void k_raster_fwd(const int32_t *__restrict__ ranges, const int32_t *__restrict__ order,
                                                   const uint2 *__restrict__ qent, const uint32_t *__restrict__ qk,
                                                   const char *__restrict__ rb, const uint64_t *__restrict__ bitmap,
                                                   const uint32_t *__restrict__ wpre, int64_t words, int W, int H,
                                                   int TX, int T, float alpha_min, float alpha_max, float t_min,
                                                   float *__restrict__ out_c, float *__restrict__ out_t,
                                                   int32_t *__restrict__ out_n)
{
    int tile, q;
    raster_block(order, tile, q);
    const int lane = threadIdx.x;
    const int px = (tile % TX) * GS_TILE + (q & 1) * 8 + (lane & 7);
    const int py = (tile / TX) * GS_TILE + (q >> 1) * 8 + (lane >> 3);
    const bool inside = px < W && py < H;
    if (__ballot(inside) == 0) return;
    const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
    const int start = ranges[tile], end = ranges[tile + 1];
    if (start >= end) {   // empty list: nothing is read (the quadrant prefix counts may be unset)
        if (inside) {
            const size_t idx = (size_t)py * W + px;
            out_c[3 * idx] = 0.0f;
            out_c[3 * idx + 1] = 0.0f;
            out_c[3 * idx + 2] = 0.0f;
            out_t[idx] = 1.0f;
            out_n[idx] = 0;
        }
        return;
    }
    const uint64_t *bq = bitmap + (int64_t)q * words;
    const uint32_t *wq = wpre + (int64_t)q * (words + 1);
    const uint32_t j0 = quad_prefix(bq, wq, (uint32_t)start), j1 = quad_prefix(bq, wq, (uint32_t)end);
    const float4 *grec = reinterpret_cast<const float4 *>(rb + reinterpret_cast<const BinsHeader *>(rb)->grec_off);
    float Tr, cr, cg, cb;
    int np;
    fwd_walk(qent, qk, grec, j0, j1, fx, fy, start, end, inside, alpha_min, alpha_max, t_min, cr, cg, cb, Tr, np);
    if (inside) {
        const size_t idx = (size_t)py * W + px;
        out_c[3 * idx] = cr;
        out_c[3 * idx + 1] = cg;
        out_c[3 * idx + 2] = cb;
        out_t[idx] = Tr;
        out_n[idx] = np;
    }
}

// sum over the image of N_p, added to *n_sum: one 64-bit atomic per block (a device-wide
// counter updated once per raster wave would serialise ~10^4 atomics on one address).
// Each thread reads four 16-byte groups of pixels, independently, when n_trav is 16-byte
// aligned; otherwise single pixels.
constexpr int kSumGroups = 4;

__global__ __launch_bounds__(256) void k_sum_ntrav(const int32_t *__restrict__ n_trav, int64_t n_px,
                                                   unsigned long long *__restrict__ n_sum)
{
    __shared__ unsigned long long part[4];
    unsigned long long acc = 0;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x, stride = (int64_t)gridDim.x * 256;
    if ((reinterpret_cast<uintptr_t>(n_trav) & 15) == 0) {
        const int4 *v = reinterpret_cast<const int4 *>(n_trav);
        const int64_t n4 = n_px >> 2;
        int4 x[kSumGroups];
#pragma unroll
        for (int u = 0; u < kSumGroups; ++u) {
            const int64_t i = t + u * stride;
            x[u] = i < n4 ? v[i] : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kSumGroups; ++u)
            acc += (unsigned long long)((uint32_t)x[u].x + (uint32_t)x[u].y) + ((uint32_t)x[u].z + (uint32_t)x[u].w);
        for (int64_t i = t + kSumGroups * stride; i < n4; i += stride) {
            const int4 y = v[i];
            acc += (unsigned long long)((uint32_t)y.x + (uint32_t)y.y) + ((uint32_t)y.z + (uint32_t)y.w);
        }
        if (t < (n_px & 3)) acc += (uint32_t)n_trav[(n4 << 2) + t];
    } else {
        for (int64_t i = t; i < n_px; i += stride) acc += (uint32_t)n_trav[i];
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_down(acc, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long s = part[0] + part[1] + part[2] + part[3];
        if (s) atomicAdd(n_sum, s);
    }
}

}  // namespace

namespace gsi {

gs_status check_raster_inputs(const gs_bins *bins, const gs_camera *cam)
{
    if (!bins) return fail(GS_ERR_INVALID_ARGUMENT, "bins is NULL");
    if (!bins->tile_ranges) return fail(GS_ERR_INVALID_ARGUMENT, "tile_ranges is NULL");
    if (!bins->raster || !aligned(bins->raster, 256))
        return fail(GS_ERR_INVALID_ARGUMENT, "raster buffer is NULL or not 256-byte aligned");
    if (bins->capacity < 0) return fail(GS_ERR_INVALID_ARGUMENT, "capacity < 0");
    (void)cam;
    return GS_OK;
}

}  // namespace gsi

extern "C" gs_status gs_raster_fwd(const gs_projected *proj, const gs_bins *bins, const gs_camera *cam,
                                   const gs_raster_params *p, float *color, float *t_final, int32_t *n_trav,
                                   unsigned long long *n_trav_sum, hipStream_t stream)
{
    using namespace gsi;
    (void)proj;   // the raster buffer carries copies of the projected records
    gs_status s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(bins, cam)) != GS_OK) return s;
    if (!color || !t_final || !n_trav) return fail(GS_ERR_INVALID_ARGUMENT, "an output pointer is NULL");
    const int TX = tiles_x(cam->width), T = TX * tiles_y(cam->height);
    // the fields read here come before the n-dependent ones; grec's offset is in the header
    const RasterLayout L = raster_layout(0, bins->capacity, T);
    const char *rb = static_cast<const char *>(bins->raster);
    k_raster_fwd<<<(unsigned)raster_grid(T), 64, 0, stream>>>(
        bins->tile_ranges, reinterpret_cast<const int32_t *>(rb + L.order),
        reinterpret_cast<const uint2 *>(rb + L.qent), reinterpret_cast<const uint32_t *>(rb + L.qk), rb,
        reinterpret_cast<const uint64_t *>(rb + L.bitmap), reinterpret_cast<const uint32_t *>(rb + L.wpre), L.words,
        cam->width, cam->height, TX, T, p->alpha_min, p->alpha_max, p->t_min, color, t_final, n_trav);
    GS_LAUNCH_CHECK("k_raster_fwd");
    if (n_trav_sum) {
        const int64_t n_px = (int64_t)cam->width * cam->height;
        const int64_t blocks = std::min<int64_t>(std::max<int64_t>(ceil_div(n_px, 256 * 4 * kSumGroups), 1), 1024);
        k_sum_ntrav<<<(unsigned)blocks, 256, 0, stream>>>(n_trav, n_px, n_trav_sum);
        GS_LAUNCH_CHECK("k_sum_ntrav");
    }
    return GS_OK;
}
