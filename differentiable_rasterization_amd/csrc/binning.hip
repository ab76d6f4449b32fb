// Tile binning and depth ordering of the tile-Gaussian intersection lists
// (ByteSplat, section 2.1: projection determines the tiles each Gaussian
// intersects and builds the tile-Gaussian list; sorting orders each tile's
// Gaussians near to far).
//
// Instead of radix-sorting 64-bit (tile | depth) keys over all K intersections,
// the Gaussians (N <= K) are sorted once by their 32-bit depth key; each then
// emits its entries in that order, and a stable sort of the entries by tile id
// (1-2 eight-bit passes for up to 65536 tiles) leaves every tile's list in
// (depth key, index) order.  Same result, roughly a quarter of the bytes.
#include "kernels.h"

namespace {

constexpr uint32_t kCulledKey = 0xFFFFFFFFu;

__global__ __launch_bounds__(256) void k_depth_keys(const int2 *__restrict__ radii, const float *__restrict__ depth,
                                                    int64_t n, uint32_t *__restrict__ keys, uint32_t *__restrict__ vals)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int2 r = radii[i];
    keys[i] = (r.x > 0 && r.y > 0) ? __float_as_uint(depth[i]) : kCulledKey;
    vals[i] = (uint32_t)i;
}

// Tile counts of the Gaussians in depth order (0 for culled ones).
__global__ __launch_bounds__(256) void k_count(const uint32_t *__restrict__ skeys, const uint32_t *__restrict__ svals,
                                               const float2 *__restrict__ means2d, const int2 *__restrict__ radii,
                                               int64_t n, int tx, int ty, uint32_t *__restrict__ cnt)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    uint32_t c = 0;
    if (skeys[j] != kCulledKey) {
        const uint32_t g = svals[j];
        const float2 m = means2d[g];
        const int2 r = radii[g];
        int x0, x1, y0, y1;
        gsd::tile_rect(m.x, m.y, r.x, r.y, tx, ty, x0, x1, y0, y1);
        c = (uint32_t)((x1 - x0) * (y1 - y0));
    }
    cnt[j] = c;
}

// Entries (tile id, Gaussian) of each Gaussian in depth order, tiles row-major.
__global__ __launch_bounds__(256) void k_emit(const uint32_t *__restrict__ svals, const uint32_t *__restrict__ cnt,
                                              const uint32_t *__restrict__ off, const float2 *__restrict__ means2d,
                                              const int2 *__restrict__ radii, int64_t n, int tx, int ty,
                                              uint32_t *__restrict__ tkeys, uint32_t *__restrict__ tvals)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n || cnt[j] == 0) return;
    const uint32_t g = svals[j];
    const float2 m = means2d[g];
    const int2 r = radii[g];
    int x0, x1, y0, y1;
    gsd::tile_rect(m.x, m.y, r.x, r.y, tx, ty, x0, x1, y0, y1);
    uint32_t p = off[j];
    for (int y = y0; y < y1; ++y)
        for (int x = x0; x < x1; ++x) {
            tkeys[p] = (uint32_t)(y * tx + x);
            tvals[p] = g;
            ++p;
        }
}

// tile_ranges[t] = first entry of tile t (entries sorted by tile); ranges[T] = K.
__global__ __launch_bounds__(256) void k_ranges(const uint32_t *__restrict__ tkeys, int64_t K, int32_t T,
                                                int32_t *__restrict__ ranges)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    const int32_t t = (int32_t)tkeys[k];
    const int32_t prev = k > 0 ? (int32_t)tkeys[k - 1] : -1;
    for (int32_t u = prev + 1; u <= t; ++u) ranges[u] = (int32_t)k;
    if (k == K - 1)
        for (int32_t u = t + 1; u <= T; ++u) ranges[u] = (int32_t)K;
}

__global__ __launch_bounds__(256) void k_keys64(const uint32_t *__restrict__ tkeys, const uint32_t *__restrict__ ids,
                                                const float *__restrict__ depth, int64_t K, uint64_t *__restrict__ keys)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    keys[k] = ((uint64_t)tkeys[k] << 32) | (uint64_t)__float_as_uint(depth[ids[k]]);
}

__global__ __launch_bounds__(256) void k_touched(const uint32_t *__restrict__ svals, const uint32_t *__restrict__ cnt,
                                                 int64_t n, int32_t *__restrict__ touched)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    touched[svals[j]] = (int32_t)cnt[j];
}

struct Layout {
    size_t dkA, dvA, dkB, dvB, cnt, off, total, tkA, tkB, tv, hist, part, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout layout(int64_t n, int64_t cap)
{
    Layout L;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
    const size_t nn = (size_t)(n > 0 ? n : 1), cc = (size_t)(cap > 0 ? cap : 1);
    L.dkA = take(4 * nn); L.dvA = take(4 * nn); L.dkB = take(4 * nn); L.dvB = take(4 * nn);
    L.cnt = take(4 * nn); L.off = take(4 * nn); L.total = take(8);
    L.tkA = take(4 * cc); L.tkB = take(4 * cc); L.tv = take(4 * cc);
    const int64_t mmax = std::max<int64_t>(n, cap);
    const int64_t hl = gsi::radix_hist_len(mmax);
    L.hist = take(4 * (size_t)hl);
    const int64_t pl = std::max(gsi::scan_partials_len(hl), gsi::scan_partials_len(mmax));
    L.part = take(4 * (size_t)pl);
    L.bytes = o;
    return L;
}

int bits_for(int64_t maxval)
{
    int b = 0;
    while (b < 63 && (int64_t(1) << b) <= maxval) ++b;
    return b;
}

}  // namespace

extern "C" size_t gs_bin_sort_workspace_bytes(int64_t n, int64_t capacity, int32_t width, int32_t height)
{
    (void)width; (void)height;
    if (n < 0 || capacity < 0) return 0;
    return layout(n, capacity).bytes;
}

extern "C" gs_status gs_bin_sort(const gs_projected *proj, int64_t n, const gs_camera *cam, gs_bins *bins,
                                 int64_t *n_isect_out, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if (!proj || !bins || !n_isect_out) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    if (n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
    if (n > (int64_t(1) << 31) - 1) return fail(GS_ERR_UNSUPPORTED, "n >= 2^31");
    if (bins->capacity < 0 || bins->capacity > 0xFFFFFFFFll)
        return fail(GS_ERR_INVALID_ARGUMENT, "capacity out of range");
    if (!bins->tile_ranges || (bins->capacity > 0 && !bins->ids))
        return fail(GS_ERR_INVALID_ARGUMENT, "ids / tile_ranges is NULL");
    const int tx = tiles_x(cam->width), ty = tiles_y(cam->height);
    const int32_t T = tx * ty;
    *n_isect_out = 0;
    if (n == 0) return fill_i32(bins->tile_ranges, (int64_t)T + 1, 0, stream);
    if (!proj->means2d || !proj->depth || !proj->radii)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected means2d / depth / radii is NULL");
    if (!aligned(proj->means2d, 8) || !aligned(proj->radii, 8))
        return fail(GS_ERR_INVALID_ARGUMENT, "means2d / radii must be 8-byte aligned");
    const Layout L = layout(n, bins->capacity);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.bytes)
        return fail(GS_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, 256-byte aligned", L.bytes);
    char *ws = static_cast<char *>(workspace);
    uint32_t *dkA = (uint32_t *)(ws + L.dkA), *dvA = (uint32_t *)(ws + L.dvA);
    uint32_t *dkB = (uint32_t *)(ws + L.dkB), *dvB = (uint32_t *)(ws + L.dvB);
    uint32_t *cnt = (uint32_t *)(ws + L.cnt), *off = (uint32_t *)(ws + L.off);
    unsigned long long *total = (unsigned long long *)(ws + L.total);
    uint32_t *tkA = (uint32_t *)(ws + L.tkA), *tkB = (uint32_t *)(ws + L.tkB), *tv = (uint32_t *)(ws + L.tv);
    uint32_t *hist = (uint32_t *)(ws + L.hist), *part = (uint32_t *)(ws + L.part);
    const float2 *m2 = reinterpret_cast<const float2 *>(proj->means2d);
    const int2 *rr = reinterpret_cast<const int2 *>(proj->radii);
    const unsigned gn = (unsigned)ceil_div(n, 256);

    // 1. Gaussians by depth key (stable, so equal keys stay in index order)
    k_depth_keys<<<gn, 256, 0, stream>>>(rr, proj->depth, n, dkA, dvA);
    GS_LAUNCH_CHECK("k_depth_keys");
    bool in_b = false;
    if ((s = radix_sort_u32(dkA, dvA, dkB, dvB, n, 32, hist, part, &in_b, stream)) != GS_OK) return s;
    const uint32_t *sk = in_b ? dkB : dkA, *sv = in_b ? dvB : dvA;

    // 2. tile counts in depth order, their exclusive scan, and the total K
    k_count<<<gn, 256, 0, stream>>>(sk, sv, m2, rr, n, tx, ty, cnt);
    GS_LAUNCH_CHECK("k_count");
    if ((s = exclusive_scan_u32(cnt, off, n, part, total, stream)) != GS_OK) return s;
    unsigned long long K = 0;
    GS_HIP(hipMemcpyAsync(&K, total, sizeof(K), hipMemcpyDeviceToHost, stream));
    GS_HIP(hipStreamSynchronize(stream));
    *n_isect_out = (int64_t)K;
    if (K > 0xFFFFFFFFull) return fail(GS_ERR_UNSUPPORTED, "more than 2^32 intersections");
    if ((int64_t)K > bins->capacity)
        return fail(GS_ERR_CAPACITY, "%llu intersections exceed the capacity %lld", K, (long long)bins->capacity);

    if (bins->tiles_touched) {
        k_touched<<<gn, 256, 0, stream>>>(sv, cnt, n, bins->tiles_touched);
        GS_LAUNCH_CHECK("k_touched");
    }
    if (K == 0) return fill_i32(bins->tile_ranges, (int64_t)T + 1, 0, stream);

    // 3. emit entries in depth order, then a stable sort by tile id
    const int tbits = std::max(1, bits_for(T - 1));
    const int passes = (tbits + 7) / 8;
    uint32_t *ev = (passes % 2 == 1) ? tv : bins->ids;     // the last pass lands in bins->ids
    uint32_t *ov = (passes % 2 == 1) ? bins->ids : tv;
    k_emit<<<gn, 256, 0, stream>>>(sv, cnt, off, m2, rr, n, tx, ty, tkA, ev);
    GS_LAUNCH_CHECK("k_emit");
    if ((s = radix_sort_u32(tkA, ev, tkB, ov, (int64_t)K, tbits, hist, part, &in_b, stream)) != GS_OK) return s;
    const uint32_t *tk = in_b ? tkB : tkA;
    if (K == 1 && ev != bins->ids) {
        // a single entry is not moved by the sort
        GS_HIP(hipMemcpyAsync(bins->ids, ev, 4, hipMemcpyDeviceToDevice, stream));
    }

    // 4. per-tile ranges, optional 64-bit keys
    const unsigned gk = (unsigned)ceil_div((int64_t)K, 256);
    k_ranges<<<gk, 256, 0, stream>>>(tk, (int64_t)K, T, bins->tile_ranges);
    GS_LAUNCH_CHECK("k_ranges");
    if (bins->keys) {
        k_keys64<<<gk, 256, 0, stream>>>(tk, bins->ids, proj->depth, (int64_t)K, bins->keys);
        GS_LAUNCH_CHECK("k_keys64");
    }
    return GS_OK;
}
