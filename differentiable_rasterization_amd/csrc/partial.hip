// Partial renders of depth slabs: over-composition along the pixel ray and its
// backward (Splaxel, sections 3.4 and 4.2 -- partial pixels of convex partitions
// aggregated in depth order reproduce the global blending order; section 4.3 --
// once the accumulated transmittance is below epsilon later partitions contribute
// nothing), and the compaction of non-zero screen-space gradient records (ByteSplat,
// section 3 Insight 4 and section 6: a record is dropped only if all of its fields
// are exactly zero, so aggregation is unchanged).
#include "kernels.h"

namespace {

constexpr int kMaxParts = 16;

struct Parts {
    const float *c[kMaxParts];
    const float *t[kMaxParts];
    float *dc[kMaxParts];
    float *dt[kMaxParts];
    int k;
};

__global__ __launch_bounds__(256) void k_composite(Parts P, int64_t n_px, float t_min, float *__restrict__ c_out,
                                                   float *__restrict__ t_out)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_px) return;
    float A = 1.0f, r = 0.0f, g = 0.0f, b = 0.0f;
    for (int k = 0; k < P.k; ++k) {
        if (A < t_min) continue;
        r = fmaf(A, P.c[k][3 * p], r);
        g = fmaf(A, P.c[k][3 * p + 1], g);
        b = fmaf(A, P.c[k][3 * p + 2], b);
        A *= P.t[k][p];
    }
    c_out[3 * p] = r;
    c_out[3 * p + 1] = g;
    c_out[3 * p + 2] = b;
    t_out[p] = A;
}

template <bool HAS_GT>
__global__ __launch_bounds__(256) void k_composite_bwd(Parts P, int64_t n_px, float t_min,
                                                       const float *__restrict__ G, const float *__restrict__ GT)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_px) return;
    float A[kMaxParts], Tk[kMaxParts];
    float a = 1.0f;
    int live = 0;   // partitions [0, live) are composited, the rest skipped
    for (int k = 0; k < P.k; ++k) {
        A[k] = a;
        if (a < t_min) break;
        Tk[k] = P.t[k][p];
        a *= Tk[k];
        live = k + 1;
    }
    const float g0 = G[3 * p], g1 = G[3 * p + 1], g2 = G[3 * p + 2];
    const float gt = HAS_GT ? GT[p] : 0.0f;
    // walk back: U = composite behind k, S = product of the T's behind k
    float u0 = 0.0f, u1 = 0.0f, u2 = 0.0f, S = 1.0f;
    for (int k = P.k - 1; k >= 0; --k) {
        if (k >= live) {
            P.dc[k][3 * p] = 0.0f;
            P.dc[k][3 * p + 1] = 0.0f;
            P.dc[k][3 * p + 2] = 0.0f;
            P.dt[k][p] = 0.0f;
            continue;
        }
        P.dc[k][3 * p] = A[k] * g0;
        P.dc[k][3 * p + 1] = A[k] * g1;
        P.dc[k][3 * p + 2] = A[k] * g2;
        P.dt[k][p] = A[k] * (u0 * g0 + u1 * g1 + u2 * g2) + A[k] * S * gt;
        const float *c = P.c[k] + 3 * p;
        u0 = fmaf(Tk[k], u0, c[0]);
        u1 = fmaf(Tk[k], u1, c[1]);
        u2 = fmaf(Tk[k], u2, c[2]);
        S *= Tk[k];
    }
}

// Bitmap words and per-block counts of Gaussians with a non-zero field.
__global__ __launch_bounds__(256) void k_compact_flags(const float *__restrict__ g2, int64_t n,
                                                       uint32_t *__restrict__ bitmap, uint32_t *__restrict__ counts)
{
    __shared__ uint32_t wc[4];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    bool nz = false;
    if (i < n) {
#pragma unroll
        for (int f = 0; f < 9; ++f) nz |= g2[(size_t)f * n + i] != 0.0f;
    }
    const uint64_t b = __ballot(nz);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t i0 = i - lane;   // first Gaussian of this wave
    if (lane == 0 && i0 < n) bitmap[i0 / 32] = (uint32_t)b;
    if (lane == 1 && i0 + 32 < n) bitmap[i0 / 32 + 1] = (uint32_t)(b >> 32);
    if (lane == 0) wc[w] = (uint32_t)__popcll(b);
    __syncthreads();
    if (threadIdx.x == 0) counts[blockIdx.x] = wc[0] + wc[1] + wc[2] + wc[3];
}

__global__ __launch_bounds__(256) void k_compact_write(const float *__restrict__ g2, int64_t n, uint32_t index_base,
                                                       const uint32_t *__restrict__ offs, uint32_t *__restrict__ rec)
{
    __shared__ uint32_t wc[4];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float v[9];
    bool nz = false;
#pragma unroll
    for (int f = 0; f < 9; ++f) {
        v[f] = i < n ? g2[(size_t)f * n + i] : 0.0f;
        nz |= v[f] != 0.0f;
    }
    const uint64_t b = __ballot(nz);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) wc[w] = (uint32_t)__popcll(b);
    __syncthreads();
    uint32_t pos = offs[blockIdx.x] + gsd::rank_below(b);
    for (int k = 0; k < w; ++k) pos += wc[k];
    if (nz) {
        uint32_t *r = rec + (size_t)pos * 10;
        r[0] = index_base + (uint32_t)i;
#pragma unroll
        for (int f = 0; f < 9; ++f) r[1 + f] = __float_as_uint(v[f]);
    }
}

// Owner-side decoding of compacted records (ByteSplat section 6.2): each record's
// partition position is mapped through the forward-communication index of its
// partition to the owner's Gaussian, and its non-zero fields are added to the owner's
// gradient planes with fp32 atomics -- a Gaussian sent to several renderers receives
// one record from each, so the adds may collide.  One block decodes 256 records of one
// partition; they are staged through LDS so the 40-byte records are read with
// coalesced dword loads.
constexpr int kDecodeRecords = 256;
constexpr int kRecordWords = 10;

struct DecodeParts {
    const uint32_t *rec[kMaxParts];
    const uint32_t *map[kMaxParts];   // NULL: identity
    uint32_t base[kMaxParts];
    uint32_t n_part[kMaxParts];
    uint32_t r[kMaxParts];
    uint32_t first_block[kMaxParts + 1];
    int k;
};

__global__ __launch_bounds__(256) void k_decode_grads(DecodeParts D, float *__restrict__ g2, uint32_t n_owner,
                                                      uint32_t *__restrict__ rejected)
{
    __shared__ uint32_t st[kDecodeRecords * kRecordWords];
    const uint32_t b = blockIdx.x;
    int p = 0;
    while (p + 1 < D.k && b >= D.first_block[p + 1]) ++p;   // uniform: kernel arguments live in SGPRs
    const uint32_t r0 = (b - D.first_block[p]) * kDecodeRecords;
    const uint32_t cnt = min((uint32_t)kDecodeRecords, D.r[p] - r0);
    const uint32_t *src = D.rec[p] + (size_t)r0 * kRecordWords;
    const int t = threadIdx.x;
#pragma unroll
    for (int w = 0; w < kRecordWords; ++w) {
        const uint32_t j = (uint32_t)(w * kDecodeRecords + t);
        if (j < cnt * kRecordWords) st[j] = src[j];
    }
    __syncthreads();
    bool bad = false;
    if ((uint32_t)t < cnt) {
        const uint32_t *rw = st + t * kRecordWords;
        const uint32_t i = rw[0] - D.base[p];   // wraps to a large value below the base
        uint32_t o = 0xFFFFFFFFu;
        if (i < D.n_part[p]) o = D.map[p] ? D.map[p][i] : i;
        if (o < n_owner) {
#pragma unroll
            for (int f = 0; f < 9; ++f) {
                const float v = __uint_as_float(rw[1 + f]);
                if (v != 0.0f) unsafeAtomicAdd(g2 + (size_t)f * n_owner + o, v);
            }
        } else {
            bad = true;
        }
    }
    const uint64_t m = __ballot(bad);
    if (rejected && m && (t & 63) == 0) atomicAdd(rejected, (uint32_t)__popcll(m));
}

gs_status fill_parts(Parts &P, const float *const *c_k, const float *const *t_k, int32_t k, int64_t n_px)
{
    using namespace gsi;
    if (k < 1 || k > kMaxParts) return fail(GS_ERR_INVALID_ARGUMENT, "k must lie in [1, 16]");
    if (n_px < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_px < 0");
    if (!c_k || !t_k) return fail(GS_ERR_INVALID_ARGUMENT, "c_k / t_k is NULL");
    P.k = k;
    for (int i = 0; i < k; ++i) {
        if (n_px > 0 && (!c_k[i] || !t_k[i])) return fail(GS_ERR_INVALID_ARGUMENT, "partition %d is NULL", i);
        P.c[i] = c_k[i];
        P.t[i] = t_k[i];
    }
    return GS_OK;
}

}  // namespace

extern "C" gs_status gs_composite_over(const float *const *c_k, const float *const *t_k, int32_t k, int64_t n_px,
                                       float t_min, float *c_out, float *t_out, hipStream_t stream)
{
    using namespace gsi;
    Parts P = {};
    gs_status s;
    if ((s = fill_parts(P, c_k, t_k, k, n_px)) != GS_OK) return s;
    if (n_px == 0) return GS_OK;
    if (!c_out || !t_out) return fail(GS_ERR_INVALID_ARGUMENT, "c_out / t_out is NULL");
    k_composite<<<(unsigned)ceil_div(n_px, 256), 256, 0, stream>>>(P, n_px, t_min, c_out, t_out);
    GS_LAUNCH_CHECK("k_composite");
    return GS_OK;
}

extern "C" gs_status gs_composite_over_bwd(const float *const *c_k, const float *const *t_k, int32_t k, int64_t n_px,
                                           float t_min, const float *dL_dc, const float *dL_dt,
                                           float *const *dL_dc_k, float *const *dL_dt_k, hipStream_t stream)
{
    using namespace gsi;
    Parts P = {};
    gs_status s;
    if ((s = fill_parts(P, c_k, t_k, k, n_px)) != GS_OK) return s;
    if (n_px == 0) return GS_OK;
    if (!dL_dc || !dL_dc_k || !dL_dt_k) return fail(GS_ERR_INVALID_ARGUMENT, "NULL gradient argument");
    for (int i = 0; i < k; ++i) {
        if (!dL_dc_k[i] || !dL_dt_k[i]) return fail(GS_ERR_INVALID_ARGUMENT, "partition gradient %d is NULL", i);
        P.dc[i] = dL_dc_k[i];
        P.dt[i] = dL_dt_k[i];
    }
    const unsigned grid = (unsigned)ceil_div(n_px, 256);
    if (dL_dt)
        k_composite_bwd<true><<<grid, 256, 0, stream>>>(P, n_px, t_min, dL_dc, dL_dt);
    else
        k_composite_bwd<false><<<grid, 256, 0, stream>>>(P, n_px, t_min, dL_dc, nullptr);
    GS_LAUNCH_CHECK("k_composite_bwd");
    return GS_OK;
}

extern "C" size_t gs_compact_workspace_bytes(int64_t n)
{
    if (n < 0) return 0;
    const int64_t nb = gsi::ceil_div(n > 0 ? n : 1, 256);
    const size_t counts = ((size_t)nb * 4 + 255) & ~size_t(255);
    const size_t part = ((size_t)gsi::scan_partials_len(nb) * 4 + 255) & ~size_t(255);
    return counts + part + 256;
}

extern "C" gs_status gs_compact_grads(const float *grads2d, int64_t n, uint32_t index_base, void *records,
                                      uint32_t *bitmap, int64_t *r_out, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream)
{
    using namespace gsi;
    if (n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
    if (!r_out) return fail(GS_ERR_INVALID_ARGUMENT, "r_out is NULL");
    *r_out = 0;
    if (n == 0) return GS_OK;
    if (n > 0xFFFFFFFFll) return fail(GS_ERR_UNSUPPORTED, "n >= 2^32");
    if (!grads2d || !records || !bitmap) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(records, 4)) return fail(GS_ERR_INVALID_ARGUMENT, "records must be 4-byte aligned");
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < gs_compact_workspace_bytes(n))
        return fail(GS_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, 256-byte aligned",
                    gs_compact_workspace_bytes(n));
    const int64_t nb = ceil_div(n, 256);
    char *ws = static_cast<char *>(workspace);
    uint32_t *counts = reinterpret_cast<uint32_t *>(ws);
    const size_t counts_bytes = ((size_t)nb * 4 + 255) & ~size_t(255);
    uint32_t *part = reinterpret_cast<uint32_t *>(ws + counts_bytes);
    const size_t part_bytes = ((size_t)scan_partials_len(nb) * 4 + 255) & ~size_t(255);
    unsigned long long *total = reinterpret_cast<unsigned long long *>(ws + counts_bytes + part_bytes);
    k_compact_flags<<<(unsigned)nb, 256, 0, stream>>>(grads2d, n, bitmap, counts);
    GS_LAUNCH_CHECK("k_compact_flags");
    gs_status s = exclusive_scan_u32(counts, counts, nb, part, total, stream);
    if (s != GS_OK) return s;
    k_compact_write<<<(unsigned)nb, 256, 0, stream>>>(grads2d, n, index_base, counts,
                                                      static_cast<uint32_t *>(records));
    GS_LAUNCH_CHECK("k_compact_write");
    unsigned long long R = 0;
    GS_HIP(hipMemcpyAsync(&R, total, sizeof(R), hipMemcpyDeviceToHost, stream));
    GS_HIP(hipStreamSynchronize(stream));
    *r_out = (int64_t)R;
    return GS_OK;
}

extern "C" gs_status gs_decode_grads(const gs_grad_records *parts, int32_t k, float *grads2d, int64_t n_owner,
                                     uint32_t *rejected, hipStream_t stream)
{
    using namespace gsi;
    if (k < 0 || k > kMaxParts) return fail(GS_ERR_INVALID_ARGUMENT, "k must lie in [0, 16]");
    if (n_owner < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_owner < 0");
    if (n_owner >= 0xFFFFFFFFll) return fail(GS_ERR_UNSUPPORTED, "n_owner >= 2^32 - 1");
    if (k > 0 && !parts) return fail(GS_ERR_INVALID_ARGUMENT, "parts is NULL");
    DecodeParts D = {};
    uint64_t blocks = 0;
    for (int i = 0; i < k; ++i) {
        const gs_grad_records &q = parts[i];
        if (q.r < 0 || q.n_part < 0) return fail(GS_ERR_INVALID_ARGUMENT, "partition %d: r or n_part < 0", i);
        if (q.r > 0xFFFFFFFFll || q.n_part > 0xFFFFFFFFll)
            return fail(GS_ERR_UNSUPPORTED, "partition %d: r or n_part >= 2^32", i);
        if (q.r > 0 && !q.records) return fail(GS_ERR_INVALID_ARGUMENT, "partition %d: records is NULL", i);
        if (!aligned(q.records, 4) || !aligned(q.owner_index, 4))
            return fail(GS_ERR_INVALID_ARGUMENT, "partition %d: records / owner_index must be 4-byte aligned", i);
        D.rec[i] = static_cast<const uint32_t *>(q.records);
        D.map[i] = q.owner_index;
        D.base[i] = q.index_base;
        D.n_part[i] = (uint32_t)q.n_part;
        D.r[i] = (uint32_t)q.r;
        D.first_block[i] = (uint32_t)blocks;
        blocks += (uint64_t)ceil_div(q.r, kDecodeRecords);
    }
    D.k = k;
    D.first_block[k] = (uint32_t)blocks;
    if (blocks == 0) return GS_OK;
    if (blocks > 0x7FFFFFFFull) return fail(GS_ERR_UNSUPPORTED, "too many records");
    if (n_owner == 0 && !rejected) return GS_OK;   // every record would be rejected, uncounted
    if (n_owner > 0 && !grads2d) return fail(GS_ERR_INVALID_ARGUMENT, "grads2d is NULL");
    if (!aligned(grads2d, 4) || !aligned(rejected, 4))
        return fail(GS_ERR_INVALID_ARGUMENT, "grads2d / rejected must be 4-byte aligned");
    k_decode_grads<<<(unsigned)blocks, 256, 0, stream>>>(D, grads2d, (uint32_t)n_owner, rejected);
    GS_LAUNCH_CHECK("k_decode_grads");
    return GS_OK;
}
