// Forward rasterization, L1 loss and backward rasterization in one kernel per 8x8
// quadrant (ByteSplat, section 4.2 "Fused Rasterization Dataflow": per tile, the forward
// pass is followed at once by the per-pixel loss gradient, which the backward pass
// consumes without a round trip through memory; the loss needs no neighbouring tile).
// Per wave:
//   1. the forward walk of Eq. 1 (raster_walk.h) gives C, T_final and N_p of its pixels,
//      stored as the image;
//   2. the L1 term of Eq. 2: d = C - C*, dL/dC = sign(d) / (3 H W) per channel, and the
//      wave's partial sum of |d| and of N_p;
//   3. the backward walk of Eq. 3 from registers (dL/dC, Z = C . dL/dC, N_p) over the same
//      records up to the furthest entry any of its pixels traversed.
// The results equal gs_raster_fwd -> gs_loss_l1 -> gs_raster_bwd_partials bit for bit
// (image, N_p, gradient slots); the loss agrees up to the order of its double-precision
// sum.  Every tile runs here: the records stream through scalar registers in batches, so
// there is no per-tile on-chip capacity to exceed and no second path.
//
// Tile budget diagnostic (ByteSplat section 5.2, Eq. 7-9): for a design that keeps a tile's records on
// chip, B = floor((M_budget - M_fixed) / M_g) records fit per tile, E_t = max(0, N_t - B)
// would have to be pruned from tile t and P_t = E_t / N_t (0 for an empty tile).
// k_tile_budget computes E_t and P_t from the tile lists and the totals.
#include <mutex>

#include "kernels.h"
#include "raster_walk.h"

namespace {

using namespace gsr;

// Records per scalar-load batch of the forward phase (as k_raster_fwd; measured: 2 records
// per batch lower the scalar registers to the backward phase's count but make the kernel
// slower, 0.427 -> 0.433 ms at 1M Gaussians 1080p).
constexpr int kFusedFwdBatch = 4;

// Per-wave partial sums: sum over the wave's pixels of |C - C*| (three channels) and of N_p.
struct FusedPartial {
    double loss;
    unsigned long long ntrav;
};

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float l1_sign(float d) { return d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f); }

// kCount: the counting instance (gs_raster_fused_l1 with walk_counts) also adds the wave's
// walked records, forward and backward, and its accepted (pixel, record) pairs to counts.
template <bool kCount>
__global__ __launch_bounds__(64) void k_raster_fused_l1(
    const int32_t *__restrict__ ranges, const int32_t *__restrict__ order, const uint2 *__restrict__ qent,
    const uint32_t *__restrict__ qk, const float4 *__restrict__ grec,
    const uint64_t *__restrict__ bitmap, const uint32_t *__restrict__ wpre, int64_t words, int W, int H, int TX,
    int T, float alpha_min, float alpha_max, float t_min, const float *__restrict__ target, float inv,
    float *__restrict__ out_c, float *__restrict__ out_t, int32_t *__restrict__ out_n,
    FusedPartial *__restrict__ part, uint32_t *__restrict__ final_ticket, const BinsHeader *__restrict__ hdr,
    float *__restrict__ qgrad, uint32_t *__restrict__ qstamp, unsigned long long *__restrict__ counts)
{
    int tile, q;
    raster_block(order, tile, q);
    if (blockIdx.x == 0 && threadIdx.x == 0) *final_ticket = 0u;   // for k_fused_final of this call
    const int slot = blockIdx.x;   // one partial per (tile, quadrant) wave
    const int lane = threadIdx.x;
    const int px = (tile % TX) * GS_TILE + (q & 1) * 8 + (lane & 7);
    const int py = (tile / TX) * GS_TILE + (q >> 1) * 8 + (lane >> 3);
    const bool inside = px < W && py < H;
    const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
    const int start = ranges[tile], end = ranges[tile + 1];
    const bool listed = start < end;   // wave-uniform
    // 1. forward
    float Tr = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f;
    int np = 0;
    uint32_t j0 = 0, j1 = 0;
    uint32_t walked = 0, taken = 0;
    const uint64_t *bq = bitmap + (int64_t)q * words;
    const uint32_t *wq = wpre + (int64_t)q * (words + 1);
    if (listed) {   // an empty list reads nothing (its quadrant prefix counts may be unset)
        j0 = quad_prefix(bq, wq, (uint32_t)start);
        j1 = quad_prefix(bq, wq, (uint32_t)end);
        fwd_walk<kFusedFwdBatch, kCount>(qent, qk, grec, j0, j1, fx, fy, start, end, inside, alpha_min, alpha_max,
                                         t_min, cr, cg, cb, Tr, np, &walked, &taken);
    }
    // 2. L1 loss and its gradient
    float G0 = 0.0f, G1 = 0.0f, G2 = 0.0f, Z = 0.0f;
    double lsum = 0.0;
    if (inside) {
        const size_t idx = (size_t)py * W + px;
        out_c[3 * idx] = cr;
        out_c[3 * idx + 1] = cg;
        out_c[3 * idx + 2] = cb;
        out_t[idx] = Tr;
        out_n[idx] = np;
        const float d0 = cr - target[3 * idx], d1 = cg - target[3 * idx + 1], d2 = cb - target[3 * idx + 2];
        G0 = l1_sign(d0) * inv;
        G1 = l1_sign(d1) * inv;
        G2 = l1_sign(d2) * inv;
        lsum = (double)fabsf(d0) + (double)fabsf(d1) + (double)fabsf(d2);
        Z = fmaf(cr, G0, fmaf(cg, G1, cb * G2));
    }
    if (!inside) np = 0;   // as the backward reads it for pixels outside the image
    const double wl = wave_sum_f64(lsum);
    const unsigned long long wn = wave_sum_u64((unsigned long long)np);
    if (lane == 0) {
        part[slot].loss = wl;
        part[slot].ntrav = wn;
    }
    // 3. backward, up to the furthest entry any of the wave's pixels traversed
    if (!listed) return;
    const int nmax = max(0, min(gsd::wave_max_i32(np), end - start));
    const uint32_t jb = quad_prefix(bq, wq, (uint32_t)(start + nmax));
    // this pixel's records: those before the first entry beyond its N_p
    const uint32_t jend = quad_prefix(bq, wq, (uint32_t)(start + np));
    if constexpr (kCount) {
        const unsigned long long tk = wave_sum_u64((unsigned long long)taken);
        if (lane == 0) {
            atomicAdd(&counts[0], (unsigned long long)walked);
            atomicAdd(&counts[1], (unsigned long long)(jb - j0));
            atomicAdd(&counts[2], tk);
        }
    }
    // the stamp of this call: the header's next epoch (k_fused_final stores it)
    bwd_walk(qent, grec, j0, jb, fx, fy, jend, G0, G1, G2, Z, alpha_min, alpha_max, next_epoch(hdr->epoch), qgrad,
             qstamp);
}

// The loss and sum_p N_p from the per-wave partials.  Each block adds kFinalSpan partials
// (four independent loads per thread, then a fixed tree) into its block sum; the block that
// finishes last (by a ticket) adds the block sums in block order and writes the results,
// so the result does not depend on which block finished last.  The ticket is cleared by
// k_raster_fused_l1 of the same call.  The last block also advances the header's epoch to
// the stamp k_raster_fused_l1 wrote (next_epoch), so the per-Gaussian sums that follow read
// this call's slots.
constexpr int kFinalSpan = 1024;

__device__ __forceinline__ void block_sum(double &l, unsigned long long &c, double *rl, unsigned long long *rn)
{
    l = wave_sum_f64(l);
    c = wave_sum_u64(c);
    if ((threadIdx.x & 63) == 0) {
        rl[threadIdx.x >> 6] = l;
        rn[threadIdx.x >> 6] = c;
    }
    __syncthreads();
    l = (rl[0] + rl[1]) + (rl[2] + rl[3]);
    c = rn[0] + rn[1] + rn[2] + rn[3];
}

__global__ __launch_bounds__(256) void k_fused_final(const FusedPartial *__restrict__ part, int n, double inv,
                                                     FusedPartial *__restrict__ block_part, uint32_t *__restrict__ ticket,
                                                     BinsHeader *__restrict__ hdr, float *__restrict__ loss,
                                                     unsigned long long *__restrict__ n_sum)
{
    __shared__ double rl[4];
    __shared__ unsigned long long rn[4];
    __shared__ bool last;
    const int base = blockIdx.x * kFinalSpan + threadIdx.x;
    double l = 0.0;
    unsigned long long c = 0;
    FusedPartial v[kFinalSpan / 256];
#pragma unroll
    for (int k = 0; k < kFinalSpan / 256; ++k) {
        const int i = base + k * 256;
        v[k] = i < n ? part[i] : FusedPartial{0.0, 0ull};
    }
#pragma unroll
    for (int k = 0; k < kFinalSpan / 256; ++k) {
        l += v[k].loss;
        c += v[k].ntrav;
    }
    block_sum(l, c, rl, rn);
    if (threadIdx.x == 0) {
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(&block_part[blockIdx.x].loss),
                           (unsigned long long)__double_as_longlong(l), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&block_part[blockIdx.x].ntrav, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
        last = atomicAdd(ticket, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    l = 0.0;
    c = 0;
    for (int b = threadIdx.x; b < (int)gridDim.x; b += 256) {
        l += __longlong_as_double((long long)__hip_atomic_load(
            reinterpret_cast<const unsigned long long *>(&block_part[b].loss), __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT));
        c += __hip_atomic_load(&block_part[b].ntrav, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    block_sum(l, c, rl, rn);
    if (threadIdx.x == 0) {
        if (loss) *loss = (float)(l * inv);
        if (n_sum && c) atomicAdd(n_sum, c);
        hdr->epoch = next_epoch(hdr->epoch);
    }
}

// ByteSplat Eq. 8 and Eq. 9 (section 5.2) per tile from the list lengths N_t; totals[0] += number of
// tiles over the budget, totals[1] += sum of E_t.
__global__ __launch_bounds__(256) void k_tile_budget(const int32_t *__restrict__ ranges, int T, int64_t budget,
                                                     int32_t *__restrict__ excess, float *__restrict__ frac,
                                                     unsigned long long *__restrict__ totals)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    unsigned long long over = 0, ex = 0;
    if (t < T) {
        const int64_t nt = (int64_t)ranges[t + 1] - ranges[t];
        const int64_t e = nt > budget ? nt - budget : 0;
        if (excess) excess[t] = (int32_t)e;
        if (frac) frac[t] = nt > 0 ? (float)((double)e / (double)nt) : 0.0f;
        over = e > 0 ? 1ull : 0ull;
        ex = (unsigned long long)e;
    }
    over = wave_sum_u64(over);
    ex = wave_sum_u64(ex);
    if ((threadIdx.x & 63) == 0 && totals && (over || ex)) {
        atomicAdd(&totals[0], over);
        atomicAdd(&totals[1], ex);
    }
}


}  // namespace

namespace gsi {
gs_status check_raster_inputs(const gs_bins *bins, const gs_camera *cam);
}

// Workspace: the per-wave partials, the per-block sums of k_fused_final and its ticket.
namespace {
struct FusedWs {
    size_t part, block_part, ticket, bytes;
    int waves, blocks;
};
FusedWs fused_ws(int32_t width, int32_t height)
{
    FusedWs w;
    w.waves = gsi::tiles_x(width) * gsi::tiles_y(height) * gsr::kQuads;
    w.blocks = (int)gsi::ceil_div(w.waves, kFinalSpan);
    w.part = 0;
    w.block_part = (size_t)w.waves * sizeof(FusedPartial);
    w.ticket = w.block_part + (size_t)w.blocks * sizeof(FusedPartial);
    w.bytes = w.ticket + 16;
    return w;
}
}  // namespace

extern "C" size_t gs_raster_fused_l1_workspace_bytes(int32_t width, int32_t height)
{
    if (width <= 0 || height <= 0) return 0;
    return fused_ws(width, height).bytes;
}

namespace {

// Both entry points: the checks, then the two launches with the workspace at wsb.
gs_status fused_checks(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam, const gs_raster_params *p,
                       const float *target, float *color, float *t_final, int32_t *n_trav,
                       unsigned long long *walk_counts)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(bins, cam)) != GS_OK) return s;
    if (!target || !color || !t_final || !n_trav) return fail(GS_ERR_INVALID_ARGUMENT, "an image pointer is NULL");
    if (walk_counts && !aligned(walk_counts, 8))
        return fail(GS_ERR_INVALID_ARGUMENT, "walk_counts must be 8-byte aligned");
    return GS_OK;
}

gs_status fused_launch(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam, const gs_raster_params *p,
                       const float *target, float *color, float *t_final, int32_t *n_trav, float *loss_out,
                       unsigned long long *n_trav_sum, unsigned long long *walk_counts, char *wsb, hipStream_t stream)
{
    using namespace gsi;
    const int TX = tiles_x(cam->width), T = TX * tiles_y(cam->height);
    const RasterLayout L = raster_layout(g->n, bins->capacity, T);
    char *rb = static_cast<char *>(bins->raster);
    BinsHeader *hdr = reinterpret_cast<BinsHeader *>(rb + L.hdr);
    const int64_t m = 3 * (int64_t)cam->width * cam->height;
    const FusedWs fw = fused_ws(cam->width, cam->height);
    FusedPartial *part = reinterpret_cast<FusedPartial *>(wsb + fw.part);
    FusedPartial *block_part = reinterpret_cast<FusedPartial *>(wsb + fw.block_part);
    uint32_t *ticket = reinterpret_cast<uint32_t *>(wsb + fw.ticket);
    auto kern = walk_counts ? k_raster_fused_l1<true> : k_raster_fused_l1<false>;
    kern<<<(unsigned)raster_grid(T), 64, 0, stream>>>(
        bins->tile_ranges, reinterpret_cast<const int32_t *>(rb + L.order),
        reinterpret_cast<const uint2 *>(rb + L.qent), reinterpret_cast<const uint32_t *>(rb + L.qk),
        reinterpret_cast<const float4 *>(rb + L.grec),
        reinterpret_cast<const uint64_t *>(rb + L.bitmap), reinterpret_cast<const uint32_t *>(rb + L.wpre), L.words,
        cam->width, cam->height, TX, T, p->alpha_min, p->alpha_max, p->t_min, target, (float)(1.0 / (double)m),
        color, t_final, n_trav, part, ticket, hdr, reinterpret_cast<float *>(rb + L.qgrad),
        reinterpret_cast<uint32_t *>(rb + L.qstamp), walk_counts);
    GS_LAUNCH_CHECK("k_raster_fused_l1");
    k_fused_final<<<(unsigned)fw.blocks, 256, 0, stream>>>(part, fw.waves, 1.0 / (double)m, block_part, ticket, hdr,
                                                          loss_out, n_trav_sum);
    GS_LAUNCH_CHECK("k_fused_final");
    return GS_OK;
}

// ------------------------------------------------------------------ without allocation
//
// The workspace of gs_raster_fused_l1_noalloc: a file-scope device array, one copy per GPU
// (the per-wave partials, the per-block sums and the ticket of an image of up to
// kNoAllocMaxWaves quadrant waves, 4096 x 4096 pixels).  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, taken once per device with that device
// current and kept in scratch_ptr.
constexpr int kNoAllocMaxWaves = 256 * 256 * gsr::kQuads;
constexpr size_t kNoAllocScratchBytes = ((size_t)kNoAllocMaxWaves * sizeof(FusedPartial) +
                                         (size_t)((kNoAllocMaxWaves + kFinalSpan - 1) / kFinalSpan) *
                                             sizeof(FusedPartial) + 16 + 255) & ~size_t(255);

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char *scratch_ptr[kMaxDevices] = {};

gs_status scratch_of_current_device(char **out)
{
    int dev = -1;
    GS_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return gsi::fail(GS_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        GS_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return gsi::fail(GS_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
        scratch_ptr[dev] = static_cast<char *>(ptr);
    }
    *out = scratch_ptr[dev];
    return GS_OK;
}

}  // namespace

extern "C" gs_status gs_raster_fused_l1(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam,
                                        const gs_raster_params *p, const float *target, float *color, float *t_final,
                                        int32_t *n_trav, float *loss_out, unsigned long long *n_trav_sum,
                                        unsigned long long *walk_counts, void *workspace, size_t workspace_bytes,
                                        hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = fused_checks(g, bins, cam, p, target, color, t_final, n_trav, walk_counts)) != GS_OK) return s;
    const size_t need = gs_raster_fused_l1_workspace_bytes(cam->width, cam->height);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need)
        return fail(GS_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, 16-byte aligned", need);
    return fused_launch(g, bins, cam, p, target, color, t_final, n_trav, loss_out, n_trav_sum, walk_counts,
                        static_cast<char *>(workspace), stream);
}

extern "C" gs_status gs_raster_fused_l1_noalloc(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam,
                                                const gs_raster_params *p, const float *target, float *color,
                                                float *t_final, int32_t *n_trav, float *loss_out,
                                                unsigned long long *n_trav_sum, unsigned long long *walk_counts,
                                                hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = fused_checks(g, bins, cam, p, target, color, t_final, n_trav, walk_counts)) != GS_OK) return s;
    const size_t need = gs_raster_fused_l1_workspace_bytes(cam->width, cam->height);
    if (need > kNoAllocScratchBytes)
        return fail(GS_ERR_UNSUPPORTED,
                    "a %d x %d image needs %zu bytes of workspace; the static scratch holds %zu (at most %d quadrant "
                    "waves, 4096 x 4096 pixels): use gs_raster_fused_l1 with a workspace",
                    cam->width, cam->height, need, kNoAllocScratchBytes, kNoAllocMaxWaves);
    char *wsb = nullptr;
    if ((s = scratch_of_current_device(&wsb)) != GS_OK) return s;
    return fused_launch(g, bins, cam, p, target, color, t_final, n_trav, loss_out, n_trav_sum, walk_counts, wsb,
                        stream);
}

extern "C" int64_t gs_tile_budget(int64_t lds_budget_bytes, int64_t fixed_bytes, int64_t bytes_per_gaussian)
{
    if (lds_budget_bytes < 0 || fixed_bytes < 0 || bytes_per_gaussian <= 0 || fixed_bytes > lds_budget_bytes) return -1;
    return (lds_budget_bytes - fixed_bytes) / bytes_per_gaussian;
}

extern "C" gs_status gs_tile_budget_report(const gs_bins *bins, const gs_camera *cam, int64_t budget,
                                           int32_t *excess, float *frac, unsigned long long *totals,
                                           hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if (!bins || !bins->tile_ranges) return fail(GS_ERR_INVALID_ARGUMENT, "bins / tile_ranges is NULL");
    if (budget < 0) return fail(GS_ERR_INVALID_ARGUMENT, "budget < 0");
    if (totals && !aligned(totals, 8)) return fail(GS_ERR_INVALID_ARGUMENT, "totals must be 8-byte aligned");
    const int T = tiles_x(cam->width) * tiles_y(cam->height);
    k_tile_budget<<<(unsigned)ceil_div(T, 256), 256, 0, stream>>>(bins->tile_ranges, T, budget, excess, frac, totals);
    GS_LAUNCH_CHECK("k_tile_budget");
    return GS_OK;
}
