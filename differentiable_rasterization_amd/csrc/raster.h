// Shared definitions of the binning's raster-ready lists and the forward / backward
// rasterization kernels.
//
// Raster-ready lists (the gs_bins.raster buffer, written by gs_bin_sort):
//   hdr    BinsHeader             the counts of the last sort: entries K, quadrant records
//                                 Q, and whether the lists fit the capacity
//   qent   [2 * capacity] uint2   for each 8x8 quadrant q of every tile (qx = q & 1,
//                                 qy = q >> 1), the entries of the tile's list whose
//                                 alpha >= alpha_min box reaches the quadrant, in list order,
//                                 as (Gaussian, gradient slot); quadrant 0's lists of all
//                                 tiles in tile order, then quadrant 1's, ...
//   qk     [2 * capacity] uint32  the tile-list index of each of those entries
//   bitmap [4][words] uint64      bit k of bitmap q is set if list entry k is in quadrant q
//   wpre   [4][words + 1] uint32  exclusive prefix count over all four bitmaps, word by
//                                 word, so the entries of tile t in quadrant q are
//                                 qent[P_q(start_t) .. P_q(end_t)), P_q(x) = wpre[q][x / 64]
//                                 + set bits of bitmap q below entry x in its word
//   order  [4 * tiles] int32      the (tile, quadrant) waves, w = tile * 4 + quadrant, by
//                                 decreasing quadrant record count (heaviest first)
//   qoff   [n + 1] uint32         first gradient slot of Gaussian g: its quadrant records
//                                 own slots qoff[g] .. qoff[g + 1], in the order of its
//                                 entries and, within an entry, of the quadrants (qoff[n] =
//                                 the number of quadrant records)
//   qgrad  [2 * capacity][9] f32  the backward's per-record partial gradients (9 fields,
//                                 36 bytes, packed), one slot per quadrant record, at the
//                                 slot index its record carries
//   grec   [n][4] float4          (last, at hdr.grec_off) the projected raster record of every
//                                 Gaussian (its three float4 words, then a fourth, unused),
//                                 copied at sort time (zeros for culled ones), so that the
//                                 raster calls read nothing outside this buffer
//   qstamp [2 * capacity] uint32  the epoch of the backward call that wrote each slot, kept
//                                 apart from the slots so that the per-Gaussian sums read only
//                                 the slots that were written; the sort sets the stamps of
//                                 slots 0 .. Q to 0, which no epoch equals
//
// Execution: one 64-lane wave per 8x8 quadrant of a 16x16 tile, one pixel per lane
// (lane & 7 = column, lane >> 3 = row).  A wave reads its contiguous run of list entries
// with vector loads and each entry's record with scalar loads, several records per load
// batch: the records are uniform across the wave, so they live in SGPRs and feed the vector
// ALU as operands, with no LDS traffic and no per-entry relevance test.
#pragma once

#include "common.h"

namespace gsr {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQuads = 4;

// Record layout (48 bytes; written per Gaussian by the projection, copied to grec by the
// binning).  With (dx, dy) = pixel centre - mean, the alpha exponent is evaluated base 2:
// o exp(-A dx^2/2 - B dx dy - C dy^2/2) = exp2(a dx^2 + b dx dy + c dy^2 + l)
// with a = -log2(e) A / 2, b = -log2(e) B, c = -log2(e) C / 2, l = log2(o).
//   p0 = (u, v, a, b)   p1 = (c, l, red, green)   p2 = (blue, index bits, rx bits, ry bits)
// with rx, ry the box half-extents as int32 bits.
// The backward recovers A = -2 ln(2) a, B = -ln(2) b, C = -2 ln(2) c and 1/o = exp2(-l).
struct Rec {
    float4 p0, p1, p2;
};
constexpr int kRecF4 = 3;   // float4 words per record
// The binning's copy of the records (grec) uses a 64-byte stride, so that the raster's
// gather of a record's first 36 bytes touches one 64-byte line (at a 48-byte stride half of
// them straddled two).
constexpr int kGRecF4 = 4;
constexpr int kGradSlot = 9;    // floats per per-record gradient slot (the 9 moment sums, packed)
constexpr int kStampWords = 1;  // uint32 words per slot stamp
// Quadrant records are stored for up to kQuadFactor * capacity (entry, quadrant) pairs
// (an entry reaches 1.4 - 2 quadrants on average); more is reported as a capacity error.
constexpr int kQuadFactor = 2;
constexpr float kLn2 = 0.69314718055994531f;

// Quadrant mask of an entry lives in bits 24..27 of its 32-bit tile key during the sort
// (tile ids use at most 24 bits and only those are sorted).
constexpr int kMaskShift = 24;
constexpr uint32_t kTileMask = (1u << kMaskShift) - 1u;

// Minimum of the quadratic form A x^2 + 2 B x y + C y^2 (positive definite) over the
// rectangle [xa, xb] x [ya, yb] of offsets from the mean: 0 if the rectangle holds the
// mean, otherwise the smallest of the four edge minima (each a clamped 1-D quadratic).
// bA = B / A and bC = B / C are passed in precomputed.
__device__ __forceinline__ float conic_rect_min(float A, float B, float C, float bA, float bC, float xa, float xb,
                                                float ya, float yb)
{
    if (xa <= 0.0f && xb >= 0.0f && ya <= 0.0f && yb >= 0.0f) return 0.0f;
    float m = INFINITY;
    const float xs[2] = {xa, xb}, ys[2] = {ya, yb};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float x = xs[e], y = fminf(fmaxf(-bC * x, ya), yb);
        m = fminf(m, fmaf(A * x, x, fmaf(2.0f * B * x, y, C * y * y)));
        const float y2 = ys[e], x2 = fminf(fmaxf(-bA * y2, xa), xb);
        m = fminf(m, fmaf(A * x2, x2, fmaf(2.0f * B * x2, y2, C * y2 * y2)));
    }
    return m;
}

// Bit q of the result is set if the alpha >= alpha_min ellipse of a Gaussian (conic A, B,
// C; alpha >= alpha_min  <=>  A dx^2 + 2 B dx dy + C dy^2 <= thr = 2 ln(o / alpha_min))
// can reach a pixel centre of 8x8 quadrant q (qx = q & 1, qy = q >> 1) of the tile with
// pixel origin (x0, y0): its minimum over the rectangle spanned by the quadrant's pixel
// centres is at most thr.  The absolute margin of 1e-3 on a form of order 10 (a 0.05 %
// band of alpha below alpha_min) keeps the test conservative against float rounding;
// entries it admits in error are rejected by the per-pixel alpha test.
__device__ __forceinline__ uint32_t quad_mask(float u, float v, float A, float B, float C, float thr, float x0, float y0)
{
    const float lim = thr + 1e-3f;
    const float bA = B / A, bC = B / C;
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float xa = x0 + 8.0f * (q & 1) + 0.5f - u, ya = y0 + 8.0f * (q >> 1) + 0.5f - v;
        if (conic_rect_min(A, B, C, bA, bC, xa, xa + 7.0f, ya, ya + 7.0f) <= lim) m |= 1u << q;
    }
    return m;
}

// Counts of the last sort, in device memory (the first bytes of the raster buffer).  When
// the lists did not fit (ok == 0) the sort leaves every tile list empty and the per-Gaussian
// gradient reduction writes zeros.  epoch: the sort sets it to 1 and every backward call
// advances it (next_epoch: never 0); the backward stamps each gradient slot it writes with
// the new epoch in qstamp, and the per-Gaussian sums take only slots whose stamp equals the
// current epoch.  The sort sets the stamps of all its slots to 0, so a slot the backward
// did not write since the sort (a record no pixel reached, a batch no pixel took) never
// matches, whatever the buffer held before: the raster buffer may be uninitialised.
// grec_off: the byte offset of grec in the raster buffer (it depends on n, which the
// forward raster call is not given).
struct BinsHeader {
    unsigned long long K, Q;   // tile entries and (entry, quadrant) records
    uint32_t ok, epoch;
    unsigned long long grec_off;
};

constexpr uint32_t kSortEpoch = 1u;   // the epoch a sort leaves in the header

// The epoch after e; 0 is skipped, since it is the stamp of a slot no backward wrote.
__device__ __forceinline__ uint32_t next_epoch(uint32_t e) { return e + 1u == 0u ? 1u : e + 1u; }

// The same test from a raster record (conic pre-scaled for exp2, l = log2 o):
// alpha >= alpha_min  <=>  a dx^2 + b dx dy + c dy^2 >= log2(alpha_min) - l, i.e. the
// positive form -a dx^2 - b dx dy - c dy^2 is at most l - log2(alpha_min).
__device__ __forceinline__ uint32_t quad_mask_rec(const float4 &p0, const float4 &p1, float log2_amin, float x0,
                                                  float y0)
{
    return quad_mask(p0.x, p0.y, -p0.z, -0.5f * p0.w, -p1.x, p1.y - log2_amin, x0, y0);
}

struct RasterLayout {
    size_t hdr, grec, qent, qk, bitmap, wpre, order, qoff, qgrad, qstamp, bytes;
    int64_t cap, words;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline RasterLayout raster_layout(int64_t n, int64_t capacity, int tiles)
{
    RasterLayout L;
    L.cap = capacity > 0 ? capacity : 1;
    L.words = (L.cap + 63) / 64;
    const size_t nn = (size_t)(n > 0 ? n : 1), q4 = (size_t)kQuadFactor * (size_t)L.cap;
    size_t o = 0;
    L.hdr = o;    o += align256(sizeof(BinsHeader));
    L.qent = o;   o += align256(q4 * 8);
    L.qk = o;     o += align256(q4 * 4);
    L.bitmap = o; o += align256((size_t)kQuads * (size_t)L.words * 8);
    L.wpre = o;   o += align256((size_t)kQuads * (size_t)(L.words + 1) * 4);
    L.order = o;  o += align256((size_t)kQuads * (size_t)(tiles > 0 ? tiles : 1) * 4);
    L.qoff = o;   o += align256((nn + 1) * 4);
    L.qgrad = o;  o += align256(q4 * kGradSlot * 4);
    L.qstamp = o; o += align256(q4 * kStampWords * 4);
    L.grec = o;   o += align256(nn * (size_t)kGRecF4 * 16);
    L.bytes = o;
    return L;
}

// ByteSplat Eq. 4 for Gaussian g: the sum of the gradient slots of its quadrant records,
// slots qoff[g] .. qoff[g + 1], added in order (none when the lists did not fit the
// capacity).  The slots hold per-record sums of the pixel moments S0 = dpower, Sx, Sy,
// Sxx, Sxy, Syy and the colour terms.  Returns whether g has any slot.
//
// A wave's 64 consecutive Gaussians own one contiguous run of slots.  The wave reads that
// run 64 slots at a time, coalesced, into its staging area in LDS (the stamps first; the
// data of a slot only if the latest backward call wrote it), and each lane then adds its
// own slots from LDS, in slot order.  All 64 lanes of the wave must call it; a lane past
// the last Gaussian passes g >= n (an empty range).
struct SlotStage {
    float4 d[3][64];   // d[k][l]: float4 k of slot c0 + l of the current chunk
    uint32_t ok[64];   // slot c0 + l was written by the latest backward call
};

// U: slots summed per step of a lane's loop.  With U > 1 the LDS reads of U slots are
// issued together and then added in slot order (the same sums); measured faster in the
// batch pass (two waves per SIMD by attribute), slower in k_grad_adam at 10 M.
template <int U = 1>
__device__ __forceinline__ bool raw_slot_sums(const BinsHeader *__restrict__ hdr, const uint32_t *__restrict__ qoff,
                                              const float4 *__restrict__ qgrad, const uint32_t *__restrict__ qstamp,
                                              int64_t g, int64_t n, SlotStage &S, float (&acc)[9])
{
    const int lane = threadIdx.x & 63;
    const bool ok = hdr->ok != 0u;
    const uint32_t epoch = hdr->epoch;
    const int64_t gc = g < n ? g : n;
    const uint32_t s0 = ok ? qoff[gc] : 0u, s1 = ok && g < n ? qoff[g + 1] : s0;
    const uint32_t w0 = __shfl(s0, 0, 64), w1 = __shfl(s1, 63, 64);   // the wave's run of slots
#pragma unroll
    for (int f = 0; f < 9; ++f) acc[f] = 0.0f;
    // Two-stage pipeline over the chunks of 64 slots: the stamps run two chunks ahead and the
    // slot data one chunk ahead, so the data of chunk c0 + 64 loads while chunk c0 is summed.
    uint32_t tn = 0u;
    if (w0 + (uint32_t)lane < w1) tn = qstamp[w0 + (uint32_t)lane];
    bool w;   // this lane's slot of the chunk in d0..d2 was written by the latest backward call
    float4 d0, d1, d2;
    {
        const uint32_t sl = w0 + (uint32_t)lane;
        w = sl < w1 && tn == epoch;   // unwritten slots are not read
        if (w) {
            const float *p = reinterpret_cast<const float *>(qgrad) + (size_t)sl * kGradSlot;
            d0 = make_float4(p[0], p[1], p[2], p[3]);
            d1 = make_float4(p[4], p[5], p[6], p[7]);
            d2 = make_float4(p[8], 0.0f, 0.0f, 0.0f);
        }
        if (sl + 64u < w1) tn = qstamp[sl + 64u];
    }
    for (uint32_t c0 = w0; c0 < w1; c0 += 64u) {
        if (w) {
            S.d[0][lane] = d0;
            S.d[1][lane] = d1;
            S.d[2][lane] = d2;
        }
        S.ok[lane] = w ? 1u : 0u;
        const uint32_t sn = c0 + 64u + (uint32_t)lane;
        w = sn < w1 && tn == epoch;
        if (w) {
            const float *p = reinterpret_cast<const float *>(qgrad) + (size_t)sn * kGradSlot;
            d0 = make_float4(p[0], p[1], p[2], p[3]);
            d1 = make_float4(p[4], p[5], p[6], p[7]);
            d2 = make_float4(p[8], 0.0f, 0.0f, 0.0f);
        }
        if (sn + 64u < w1) tn = qstamp[sn + 64u];
        __builtin_amdgcn_wave_barrier();
        const uint32_t lo = s0 > c0 ? s0 : c0, hi = s1 < c0 + 64u ? s1 : c0 + 64u;
        if constexpr (U == 1) {
            for (uint32_t x = lo; x < hi; ++x) {
                const uint32_t l = x - c0;
                if (S.ok[l]) {
                    const float4 a = S.d[0][l], b = S.d[1][l], c = S.d[2][l];
                    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
                    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
                    acc[8] += c.x;
                }
            }
        } else {
            for (uint32_t x = lo; x < hi; x += (uint32_t)U) {
                float4 a[U], b[U], c[U];
                bool take[U];
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const uint32_t l = min(x - c0 + (uint32_t)j, 63u);
                    take[j] = x + (uint32_t)j < hi && S.ok[l] != 0u;
                    a[j] = S.d[0][l];
                    b[j] = S.d[1][l];
                    c[j] = S.d[2][l];
                }
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    if (take[j]) {
                        acc[0] += a[j].x; acc[1] += a[j].y; acc[2] += a[j].z; acc[3] += a[j].w;
                        acc[4] += b[j].x; acc[5] += b[j].y; acc[6] += b[j].z; acc[7] += b[j].w;
                        acc[8] += c[j].x;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    return s1 > s0;
}

// The screen-space gradients (u, v, A, B, C, o, r, g, b) from the moment sums, with the
// Gaussian's own conic and opacity as its raster record holds them (conic pre-scaled by
// -log2(e)/2, l = log2 o):
//   A = -2 ln2 a, B = -ln2 b, C = -2 ln2 c,
//   du = A Sx + B Sy, dv = B Sx + C Sy, dA = -Sxx/2, dB = -Sxy, dC = -Syy/2, do = S0 2^-l.
__device__ __forceinline__ void moments_to_grads(const float (&acc)[9], float a, float b, float c, float l,
                                                 float (&out)[9])
{
    const float A = -2.0f * kLn2 * a, B = -kLn2 * b, C = -2.0f * kLn2 * c;
    out[0] = fmaf(A, acc[1], B * acc[2]);
    out[1] = fmaf(B, acc[1], C * acc[2]);
    out[2] = -0.5f * acc[3];
    out[3] = -acc[4];
    out[4] = -0.5f * acc[5];
    out[5] = acc[0] * __builtin_amdgcn_exp2f(-l);
    out[6] = acc[6];
    out[7] = acc[7];
    out[8] = acc[8];
}

// Both steps, the record read from rec[g]; a Gaussian without records (culled) gets zeros
// and its record is not read.  Called by all 64 lanes of the wave (see raw_slot_sums).
__device__ __forceinline__ void sum_slots(const BinsHeader *__restrict__ hdr, const uint32_t *__restrict__ qoff,
                                          const float4 *__restrict__ qgrad, const uint32_t *__restrict__ qstamp,
                                          const float4 *__restrict__ rec, int64_t g, int64_t n, SlotStage &S,
                                          float (&out)[9])
{
    float acc[9];
    float a = 0.0f, b = 0.0f, c = 0.0f, l = 0.0f;
    if (raw_slot_sums(hdr, qoff, qgrad, qstamp, g, n, S, acc)) {
        const float4 p0 = rec[kRecF4 * (size_t)g], p1 = rec[kRecF4 * (size_t)g + 1];
        a = p0.z; b = p0.w; c = p1.x; l = p1.y;
    }
    moments_to_grads(acc, a, b, c, l, out);
}

// Number of entries below x (0 <= x <= K) that belong to quadrant q: the position in
// quadrant q's lists (qent) of the first record at or after entry x.  bq = bitmap + q * words,
// wq = wpre + q * (words + 1).
__device__ __forceinline__ uint32_t quad_prefix(const uint64_t *__restrict__ bq, const uint32_t *__restrict__ wq,
                                                uint32_t x)
{
    const uint32_t w = x >> 6, r = x & 63u;
    uint32_t p = wq[w];
    if (r) p += (uint32_t)__popcll(bq[w] & ((1ull << r) - 1ull));
    return p;
}

// Launch geometry shared by the raster kernels: one single-wave block per (tile, quadrant),
// block b running wave order[b], so the heaviest waves start first; consecutive blocks go
// to the 8 XCDs in turn (block b runs on XCD b mod 8), so heavy waves, which cluster
// spatially, spread over the chip.
inline int64_t raster_grid(int tiles) { return (int64_t)kQuads * tiles; }

__device__ __forceinline__ void raster_block(const int32_t *__restrict__ order, int &tile, int &quad)
{
    const int w = order[blockIdx.x];
    tile = w >> 2;
    quad = w & 3;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 exponent of a record at pixel offset (dx, dy), as dx (a dx + b dy) + (c dy^2 + l):
// two multiplies and three FMAs.  Both raster kernels evaluate it this way, so the
// backward recomputes the forward's alpha bit for bit.
__device__ __forceinline__ float exponent(const float4 &p0, const float4 &p1, float dx, float dy)
{
    return fmaf(dx, fmaf(p0.z, dx, p0.w * dy), fmaf(p1.x * dy, dy, p1.y));
}

}  // namespace gsr
