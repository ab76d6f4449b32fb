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
#include <cmath>

#include "kernels.h"
#include "raster.h"

namespace {

constexpr uint32_t kCulledKey = 0xFFFFFFFFu;

// ------------------------------------------------------------------ block-cooperative entries
//
// A block takes 256 Gaussians and walks their tile entries together, 256 entries per
// round, so that a Gaussian covering many tiles does not hold up the lanes of Gaussians
// covering few, and consecutive lanes produce consecutive entries.  Entry e of the block
// belongs to the Gaussian o with off[o] <= e < off[o + 1] (block-local offsets in tile
// row-major order); its quadrant mask is tested from o's record.

struct Coop {
    uint32_t off[257];        // block-local exclusive offsets of the Gaussians' entries; off[256] = total
    float4 p0[256], p1[256];  // the Gaussians' raster records (centre, conic, opacity)
    int4 rect[256];           // first tile column and row, width in tiles, Gaussian index
    uint32_t qbase[256];      // first gradient slot of the Gaussian (emit only)
    uint32_t qacc[256];       // quadrant records of the Gaussian's entries taken so far
    uint32_t scan[256];       // inclusive scan of the current round's per-entry record counts
    uint32_t wsum[4];
};

// Inclusive scan of one value per thread over the 256-thread block.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *wsum)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t pre = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (k < w) pre += wsum[k];
    __syncthreads();
    return pre + x;
}

// Loads Gaussian t of the block (valid: it is listed; otherwise it has no entries) into
// the shared state and sets the block-local offsets.  Returns the block's entry count.
// STRIDE: float4 words per record in rec (the projection's 3, or 4 for the binning's 64-byte
// copy).  copy (may be NULL): receives the Gaussian's record (its three float4 words).
template <int STRIDE>
__device__ __forceinline__ uint32_t coop_load(Coop &S, bool valid, uint32_t g, const float4 *__restrict__ rec,
                                              int tx, int ty, uint32_t &c_out, float4 *__restrict__ copy = nullptr)
{
    const int t = threadIdx.x;
    uint32_t c = 0;
    float4 p0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), p1 = p0, p2 = p0;
    int x0 = 0, w = 1;
    int y0 = 0;
    if (valid) {
        p0 = rec[STRIDE * (size_t)g];
        p1 = rec[STRIDE * (size_t)g + 1];
        p2 = rec[STRIDE * (size_t)g + 2];
        int x1, y1;
        gsd::tile_rect(p0.x, p0.y, __float_as_int(p2.z), __float_as_int(p2.w), tx, ty, x0, x1, y0, y1);
        if (x1 > x0 && y1 > y0) {
            c = (uint32_t)((x1 - x0) * (y1 - y0));
            w = x1 - x0;
        }
    }
    if (copy) {
        copy[0] = p0;
        copy[1] = p1;
        copy[2] = p2;
    }
    const uint32_t incl = block_incl_scan(c, S.wsum);
    S.off[t] = incl - c;
    if (t == 255) S.off[256] = incl;
    S.p0[t] = p0;
    S.p1[t] = p1;
    S.rect[t] = make_int4(x0, y0, w, (int)g);
    S.qacc[t] = 0u;
    c_out = c;
    __syncthreads();
    return S.off[256];
}

// One round of entries e0 .. e0 + 255 (e = e0 + threadIdx.x).  For a real entry (e < C):
// its Gaussian o (block-local), tile (x, y), quadrant mask qm and, in slot_in, the number
// of quadrant records of o's earlier entries (all rounds).  Advances S.qacc.
struct CoopEntry {
    bool real;
    int o, x, y;
    uint32_t qm, slot_in;
};

__device__ __forceinline__ CoopEntry coop_round(Coop &S, uint32_t e0, uint32_t C, float log2_amin)
{
    const int t = threadIdx.x;
    const uint32_t e = e0 + (uint32_t)t;
    CoopEntry E{e < C, 0, 0, 0, 0u, 0u};
    if (E.real) {
        int o = 0;   // the last Gaussian whose offset is <= e (those with no entries share the next one's)
#pragma unroll
        for (int step = 128; step > 0; step >>= 1)
            if (S.off[o + step] <= e) o += step;
        const int4 R = S.rect[o];
        const uint32_t local = e - S.off[o];
        const uint32_t row = local / (uint32_t)R.z;
        E.o = o;
        E.x = R.x + (int)(local - row * (uint32_t)R.z);
        E.y = R.y + (int)row;
        E.qm = gsr::quad_mask_rec(S.p0[o], S.p1[o], log2_amin, (float)(E.x * GS_TILE), (float)(E.y * GS_TILE));
    }
    const uint32_t pc = (uint32_t)__popc(E.qm);
    const uint32_t incl = block_incl_scan(pc, S.wsum);
    S.scan[t] = incl;
    __syncthreads();
    uint32_t upd = 0;
    bool last = false;
    if (E.real) {
        const uint32_t o_begin = S.off[E.o], o_end = S.off[E.o + 1];
        const uint32_t first = (o_begin > e0 ? o_begin : e0) - e0;   // o's first entry of this round
        const uint32_t before = first ? S.scan[first - 1] : 0u;
        E.slot_in = S.qacc[E.o] + (incl - pc - before);
        const uint32_t round_end = min(min(o_end, e0 + 256u), C);
        last = e + 1 == round_end;   // o's last entry of this round
        upd = incl - before;
    }
    __syncthreads();
    if (last) S.qacc[E.o] += upd;
    __syncthreads();
    return E;
}

// The counting half of coop_round: each entry adds its quadrant-record count to its
// Gaussian's total (LDS atomics; the sum does not depend on their order, so no scan and no
// barrier per round).  The caller synchronises before reading S.qacc.
__device__ __forceinline__ void coop_count_round(Coop &S, uint32_t e0, uint32_t C, float log2_amin)
{
    const uint32_t e = e0 + (uint32_t)threadIdx.x;
    if (e >= C) return;
    int o = 0;
#pragma unroll
    for (int step = 128; step > 0; step >>= 1)
        if (S.off[o + step] <= e) o += step;
    const int4 R = S.rect[o];
    const uint32_t local = e - S.off[o];
    const uint32_t row = local / (uint32_t)R.z;
    const int x = R.x + (int)(local - row * (uint32_t)R.z), y = R.y + (int)row;
    const uint32_t qm =
        gsr::quad_mask_rec(S.p0[o], S.p1[o], log2_amin, (float)(x * GS_TILE), (float)(y * GS_TILE));
    if (qm) atomicAdd(&S.qacc[o], (uint32_t)__popc(qm));
}

// Depth keys (culled Gaussians last) in index order, with the values tile count << 32 |
// index, each Gaussian's quadrant-record count (qcnt [n + 1], qcnt[n] = 0, so that its
// exclusive scan ends with the total), optionally the tile counts for the caller
// (touched), and the copy of every Gaussian's raster record that the raster calls read
// (grec, 64-byte stride; zeros for culled ones); also clears the scans' look-back state
// for this sort (zero: zero_words uint32).
__global__ __launch_bounds__(256) void k_keys_count(const int2 *__restrict__ radii, const float *__restrict__ depth,
                                                    const float4 *__restrict__ rec, float log2_amin, int64_t n,
                                                    int tx, int ty, uint32_t *__restrict__ keys,
                                                    uint64_t *__restrict__ vals, uint32_t *__restrict__ qcnt,
                                                    int32_t *__restrict__ touched, uint32_t *__restrict__ zero,
                                                    int64_t zero_words, float4 *__restrict__ grec)
{
    __shared__ Coop S;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t z = i; z < zero_words; z += (int64_t)gridDim.x * blockDim.x) zero[z] = 0u;
    if (i == 0) qcnt[n] = 0u;
    bool vis = false;
    if (i < n) {
        const int2 r = radii[i];
        vis = r.x > 0 && r.y > 0;
        keys[i] = vis ? __float_as_uint(depth[i]) : kCulledKey;
    }
    uint32_t c;
    const uint32_t C = coop_load<gsr::kRecF4>(S, vis, (uint32_t)i, rec, tx, ty, c,
                                              i < n ? grec + gsr::kGRecF4 * (size_t)i : nullptr);
    for (uint32_t e0 = 0; e0 < C; e0 += 256u) coop_count_round(S, e0, C, log2_amin);
    __syncthreads();
    if (i < n) {
        vals[i] = ((uint64_t)c << 32) | (uint64_t)i;
        qcnt[i] = S.qacc[threadIdx.x];
        if (touched) touched[i] = (int32_t)c;
    }
}

// Capacity the lists of K entries and Q quadrant records need.
__device__ __host__ __forceinline__ unsigned long long need_capacity(unsigned long long K, unsigned long long Q)
{
    const unsigned long long qc = (Q + gsr::kQuadFactor - 1) / gsr::kQuadFactor;
    return K > qc ? K : qc;
}

// Entries of the Gaussians in depth order (block b: depth ranks 256 b ..; svals, or
// svals_b when *sel != 0: tile count << 32 | Gaussian), tiles row-major; off: exclusive
// scan of the tile counts in depth order.  Entry p gets the key
// tile | quadrant mask << 24 (the mask rides in bits the tile sort never looks at) and the
// value (gradient slot of its first quadrant record) << 32 | its Gaussian, carried through
// the tile sort.  Gaussian g's quadrant records own slots qoff[g] .. qoff[g + 1], in the
// order of its entries and, within an entry, of the quadrants.  The records are gathered in
// depth order from the 64-byte-aligned copy grec (one aligned run per Gaussian).
__global__ __launch_bounds__(256) void k_emit(const uint64_t *__restrict__ svals, const uint64_t *__restrict__ svals_b,
                                              const uint32_t *__restrict__ sel, const uint32_t *__restrict__ off,
                                              const uint32_t *__restrict__ qoff, const float4 *__restrict__ grec,
                                              float log2_amin, int64_t n, int tx,
                                              int ty, const unsigned long long *__restrict__ tot, int64_t cap,
                                              unsigned long long grec_off,
                                              unsigned long long *__restrict__ klen, gsr::BinsHeader *__restrict__ hdr,
                                              int64_t *__restrict__ counts, uint32_t *__restrict__ tkeys,
                                              uint64_t *__restrict__ tvals)
{
    __shared__ Coop S;
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const unsigned long long K = tot[0], Q = tot[1];
    const bool ok = need_capacity(K, Q) <= (unsigned long long)cap;
    if (j == 0) {
        *klen = ok ? K : 0ull;
        hdr->K = K;
        hdr->Q = Q;
        hdr->ok = ok ? 1u : 0u;
        hdr->epoch = gsr::kSortEpoch;   // the qoff scan zeroed the stamps of slots 0 .. Q
        hdr->grec_off = grec_off;
        if (counts) {
            counts[0] = (int64_t)K;
            counts[1] = ok ? 0 : (int64_t)need_capacity(K, Q);
        }
    }
    if (!ok) return;   // the whole block agrees
    const int64_t j0 = (int64_t)blockIdx.x * blockDim.x;
    if (sel && *sel) svals = svals_b;
    const uint64_t sv = j < n ? svals[j] : 0ull;
    const bool listed = (sv >> 32) != 0u;   // culled Gaussians and those off the image have no tiles
    const uint32_t g = (uint32_t)sv;
    uint32_t c;
    const uint32_t C = coop_load<gsr::kGRecF4>(S, listed, g, grec, tx, ty, c);
    if (C == 0) return;
    S.qbase[threadIdx.x] = listed ? qoff[g] : 0u;
    const uint64_t base = off[j0];
    __syncthreads();
    for (uint32_t e0 = 0; e0 < C; e0 += 256u) {
        const CoopEntry E = coop_round(S, e0, C, log2_amin);
        const uint64_t p = base + e0 + threadIdx.x;
        if (E.real && p < (uint64_t)cap) {   // p < K <= cap; the test keeps a bug from writing out of bounds
            const uint32_t slot = S.qbase[E.o] + E.slot_in;
            tkeys[p] = (uint32_t)(E.y * tx + E.x) | (E.qm << gsr::kMaskShift);
            tvals[p] = ((uint64_t)slot << 32) | (uint32_t)S.rect[E.o].w;
        }
    }
}

// Each wave of the two passes below takes kWaveWords consecutive 64-entry words, with all
// of its loads issued before any use (the passes are latency-bound).
constexpr int kWaveWords = 4;

// Finishes the sorted lists in one pass over the entries: the Gaussian index of each
// entry (only with tvals != NULL; the tile sort's last pass writes them otherwise),
// tile_ranges[t] = first entry of tile t (entries are sorted by tile; ranges[T] = K), and
// the quadrant bitmaps with their per-word bit counts (one 64-bit word per 64
// entries and quadrant).  Every word of the bitmaps and of `wcnt` [4][words + 1] is written
// (zero past the entries); the exclusive scan of wcnt gives the positions of the quadrant
// records.  The launch covers max(words, ceil((T + 1) / 64)) words; K is read on the device.
__global__ __launch_bounds__(256) void k_finish(const uint32_t *__restrict__ tkeys, const uint64_t *__restrict__ tvals,
                                                const unsigned long long *__restrict__ klen, int32_t T,
                                                uint32_t *__restrict__ ids, int32_t *__restrict__ ranges,
                                                int64_t words, uint64_t *__restrict__ bitmap,
                                                uint32_t *__restrict__ wcnt)
{
    const int lane = threadIdx.x & 63;
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kWaveWords;   // first word of the wave
    const int64_t K = (int64_t)*klen;
    if (w0 == 0 && lane < gsr::kQuads) wcnt[(int64_t)lane * (words + 1) + words] = 0u;
    uint32_t key[kWaveWords], prev[kWaveWords];
    uint64_t tv[kWaveWords];
#pragma unroll
    for (int i = 0; i < kWaveWords; ++i) {
        const int64_t k = (w0 + i) * 64 + lane;
        const int64_t kc = k < K ? k : K - 1, kp = kc > 0 ? kc - 1 : 0;   // clamped: loads stay in range
        key[i] = K > 0 ? tkeys[kc] : 0u;
        prev[i] = K > 0 ? tkeys[kp] : 0u;
        tv[i] = K > 0 && tvals ? tvals[kc] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < kWaveWords; ++i) {
        const int64_t k = (w0 + i) * 64 + lane;
        if (K == 0 && k <= T) ranges[k] = 0;   // no entries (or lists that did not fit): all lists empty
        uint32_t qm = 0;
        if (k < K) {
            const int32_t t = (int32_t)(key[i] & gsr::kTileMask);
            qm = key[i] >> gsr::kMaskShift;
            if (tvals) ids[k] = (uint32_t)tv[i];
            const int32_t pt = k > 0 ? (int32_t)(prev[i] & gsr::kTileMask) : -1;
            for (int32_t u = pt + 1; u <= t; ++u) ranges[u] = (int32_t)k;
            if (k == K - 1)
                for (int32_t u = t + 1; u <= T; ++u) ranges[u] = (int32_t)K;
        }
        const int64_t wd = w0 + i;
#pragma unroll
        for (int q = 0; q < gsr::kQuads; ++q) {
            const uint64_t b = __ballot((qm >> q) & 1u);
            if (lane == 0 && wd < words) {
                bitmap[(int64_t)q * words + wd] = b;
                wcnt[(int64_t)q * (words + 1) + wd] = (uint32_t)__popcll(b);
            }
        }
    }
}

// Writes every list entry into the list of each quadrant its box reaches, at the position
// given by the scanned bit counts: (Gaussian, gradient slot) to qent and the entry's
// tile-list index to qk.
// Blocks reach the 8 XCDs round-robin (block b on XCD b % 8).  The first `active` blocks
// are renumbered so that each XCD takes one contiguous run of them: neighbouring tiles'
// entries then share one L2.  Returns -1 for blocks past `active`.
__device__ __forceinline__ int64_t xcd_contiguous_block(int64_t active)
{
    const int64_t b = blockIdx.x;
    if (b >= active) return -1;
    const int64_t x = b % gsi::kXcds, per = active / gsi::kXcds, rem = active % gsi::kXcds;
    return x * per + (x < rem ? x : rem) + b / gsi::kXcds;
}

__global__ __launch_bounds__(256) void k_quad_lists(const uint32_t *__restrict__ tkeys, const uint64_t *__restrict__ tvals,
                                                    const unsigned long long *__restrict__ klen, int64_t words,
                                                    const uint32_t *__restrict__ wpre, uint2 *__restrict__ qent,
                                                    uint32_t *__restrict__ qk)
{
    constexpr int64_t kBlockEntries = 4 * 64 * kWaveWords;
    const int64_t K = (int64_t)*klen;
    const int64_t blk = xcd_contiguous_block((K + kBlockEntries - 1) / kBlockEntries);
    if (blk < 0) return;
    const int lane = threadIdx.x & 63;
    const int64_t w0 = (blk * 4 + (threadIdx.x >> 6)) * kWaveWords;   // first word of the wave
    if (w0 * 64 >= K) return;   // the whole wave lies past the lists
    // The entries of one 64-entry word that belong to list q are one run that starts at the
    // scanned count of that word: lane 4 i + q loads it for word w0 + i and list q.
    static_assert(gsr::kQuads == 4 && 4 * kWaveWords <= 64, "one lookup lane per word and quadrant");
    uint32_t start = 0;
    if (lane < 4 * kWaveWords && w0 + (lane >> 2) < words)
        start = wpre[(int64_t)(lane & 3) * (words + 1) + w0 + (lane >> 2)];
    uint32_t key[kWaveWords];
    uint64_t tv[kWaveWords];
#pragma unroll
    for (int i = 0; i < kWaveWords; ++i) {
        const int64_t k = (w0 + i) * 64 + lane;
        const int64_t kc = k < K ? k : K - 1;   // clamped: loads stay in range
        key[i] = tkeys[kc];
        tv[i] = tvals[kc];
    }
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < kWaveWords; ++i) {
        const int64_t k = (w0 + i) * 64 + lane;
        const uint32_t qm = k < K ? key[i] >> gsr::kMaskShift : 0u;
        const uint32_t g = (uint32_t)tv[i];
        uint32_t slot = (uint32_t)(tv[i] >> 32);
#pragma unroll
        for (int q = 0; q < gsr::kQuads; ++q) {
            const uint64_t bal = __ballot((qm >> q) & 1u);
            const uint32_t pos0 = __shfl(start, 4 * i + q, 64);
            if ((qm >> q) & 1u) {
                const uint32_t pos = pos0 + (uint32_t)__popcll(bal & below);
                qent[pos] = make_uint2(g, slot++);
                qk[pos] = (uint32_t)k;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_keys64(const uint32_t *__restrict__ tkeys, const uint32_t *__restrict__ ids,
                                                const float *__restrict__ depth,
                                                const unsigned long long *__restrict__ klen, uint64_t *__restrict__ keys)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= (int64_t)*klen) return;
    keys[k] = ((uint64_t)(tkeys[k] & gsr::kTileMask) << 32) | (uint64_t)__float_as_uint(depth[ids[k]]);
}

// The raster kernels run one wave per (tile, quadrant), in the order `order` gives (entry
// w = tile * 4 + quadrant): waves by decreasing length of their quadrant record list,
// bucketed four buckets per octave (the order within a bucket is arbitrary), so that the
// longest lists start first and the short ones fill in behind them.  Two passes over the
// waves: bucket and count (global histogram), then place.  whist and wcur [kWaveBuckets]
// must be zero before the first pass.
constexpr int kWaveBuckets = 129;   // 0: empty; 1 + 4 log2(len), 1..128

__device__ __forceinline__ uint32_t wave_bucket(uint32_t len)
{
    if (len == 0) return 0u;
    return (__float_as_uint((float)len) >> 21) - (127u << 2) + 1u;   // exponent and two mantissa bits
}

__device__ __forceinline__ uint32_t wave_len(const int32_t *__restrict__ ranges, const uint64_t *__restrict__ bitmap,
                                             const uint32_t *__restrict__ wpre, int64_t words, uint32_t w)
{
    const int t = (int)(w >> 2), q = (int)(w & 3u);
    const int start = ranges[t], end = ranges[t + 1];
    if (start >= end) return 0u;   // (the prefix counts of an empty list may be unset)
    const uint64_t *bq = bitmap + (int64_t)q * words;
    const uint32_t *wq = wpre + (int64_t)q * (words + 1);
    return gsr::quad_prefix(bq, wq, (uint32_t)end) - gsr::quad_prefix(bq, wq, (uint32_t)start);
}

__global__ __launch_bounds__(256) void k_wave_hist(const int32_t *__restrict__ ranges, const uint64_t *__restrict__ bitmap,
                                                   const uint32_t *__restrict__ wpre, int64_t words, uint32_t waves,
                                                   uint8_t *__restrict__ wb, uint32_t *__restrict__ whist)
{
    __shared__ uint32_t h[kWaveBuckets];
    for (int i = threadIdx.x; i < kWaveBuckets; i += 256) h[i] = 0;
    __syncthreads();
    const uint32_t w = blockIdx.x * 256 + threadIdx.x;
    if (w < waves) {
        const uint32_t bk = wave_bucket(wave_len(ranges, bitmap, wpre, words, w));
        wb[w] = (uint8_t)bk;
        atomicAdd(&h[bk], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kWaveBuckets; i += 256)
        if (h[i]) atomicAdd(&whist[i], h[i]);
}

__global__ __launch_bounds__(256) void k_wave_place(const uint8_t *__restrict__ wb, uint32_t waves,
                                                    const uint32_t *__restrict__ whist, uint32_t *__restrict__ wcur,
                                                    int32_t *__restrict__ order)
{
    __shared__ uint32_t first[kWaveBuckets];   // first position of each bucket (heaviest first)
    __shared__ uint32_t h[kWaveBuckets];
    if (threadIdx.x == 0) {
        uint32_t acc = 0;
        for (int b = kWaveBuckets - 1; b >= 0; --b) {
            first[b] = acc;
            acc += whist[b];
        }
    }
    for (int i = threadIdx.x; i < kWaveBuckets; i += 256) h[i] = 0;
    __syncthreads();
    const uint32_t w = blockIdx.x * 256 + threadIdx.x;
    uint32_t bk = 0, rank = 0;
    if (w < waves) {
        bk = wb[w];
        rank = atomicAdd(&h[bk], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kWaveBuckets; i += 256)
        if (h[i]) h[i] = first[i] + atomicAdd(&wcur[i], h[i]);   // this block's run in the bucket
    __syncthreads();
    if (w < waves) order[h[bk] + rank] = (int32_t)w;
}

// The waves in index order (every list empty).
__global__ __launch_bounds__(256) void k_wave_identity(uint32_t waves, int32_t *__restrict__ order)
{
    const uint32_t w = blockIdx.x * 256 + threadIdx.x;
    if (w < waves) order[w] = (int32_t)w;
}

// Counts of an empty scene (n = 0).
__global__ void k_bins_empty(gsr::BinsHeader *__restrict__ hdr, int64_t *__restrict__ counts,
                             unsigned long long grec_off)
{
    hdr->K = 0;
    hdr->Q = 0;
    hdr->ok = 1u;
    hdr->epoch = gsr::kSortEpoch;
    hdr->grec_off = grec_off;
    if (counts) {
        counts[0] = 0;
        counts[1] = 0;
    }
}

struct Layout {
    // zero region (cleared by k_keys_count at the start of every sort): tickets and
    // look-back status words of the scans
    size_t zero, tickets, xf, whist, stD, stT, scC, scQ, scW, zero_bytes;
    size_t dkA, dvA, dkB, dvB, qcnt, doff, total, klen, tkA, tkB, tvA, tvB, hist, wb, bytes;
    int tbits;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int bits_for(int64_t maxval);

// tickets: 0-3 depth sort passes, 4-6 tile sort passes, 8 tile counts, 9 quadrant counts,
// 10 quadrant bit counts
constexpr int kTkDepth = 0, kTkTile = 4, kTkCnt = 8, kTkQcnt = 9, kTkWpre = 10;

Layout layout(int64_t n, int64_t cap, int32_t tiles)
{
    Layout L;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
    const size_t nn = (size_t)(n > 0 ? n : 1), cc = (size_t)(cap > 0 ? cap : 1);
    L.tbits = std::max(1, bits_for((int64_t)tiles - 1));
    const int64_t nw = gsr::kQuads * (gsr::raster_layout(n, cap, 1).words + 1);
    L.zero = o;
    L.tickets = take(16 * 4);
    L.xf = take(4 * gsi::kRadixXfWords);   // the depth sort's key range reduction
    L.whist = take(2 * 4 * kWaveBuckets);   // wave-order histogram, then placement cursors
    L.stD = take(8 * (size_t)gsi::radix_scan_status_len((int64_t)nn, 32));
    L.stT = take(8 * (size_t)gsi::radix_scan_status_len((int64_t)cc, L.tbits));
    L.scC = take(8 * (size_t)gsi::lb_scan_tiles((int64_t)nn));
    L.scQ = take(8 * (size_t)gsi::lb_scan_tiles((int64_t)nn + 1));
    L.scW = take(8 * (size_t)gsi::lb_scan_tiles(nw));
    L.zero_bytes = o - L.zero;
    L.dkA = take(4 * nn); L.dvA = take(8 * nn); L.dkB = take(4 * nn); L.dvB = take(8 * nn);
    L.qcnt = take(4 * (nn + 1)); L.doff = take(4 * nn);
    L.total = take(16);   // K, then the quadrant records
    L.klen = take(8);     // K if the lists fit, else 0
    L.tkA = take(4 * cc); L.tkB = take(4 * cc); L.tvA = take(8 * cc); L.tvB = take(8 * cc);
    L.hist = take(4 * (size_t)gsi::radix_hist_len(std::max<int64_t>((int64_t)nn, (int64_t)cc)));
    L.wb = take((size_t)gsr::kQuads * (size_t)(tiles > 0 ? tiles : 1));   // bucket of each raster wave
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

extern "C" size_t gs_bins_raster_bytes(int64_t n, int64_t capacity, int32_t width, int32_t height)
{
    if (n < 0 || capacity < 0 || width <= 0 || height <= 0) return 0;
    return gsr::raster_layout(n, capacity, gsi::tiles_x(width) * gsi::tiles_y(height)).bytes;
}

extern "C" size_t gs_bin_sort_workspace_bytes(int64_t n, int64_t capacity, int32_t width, int32_t height)
{
    if (n < 0 || capacity < 0 || width <= 0 || height <= 0) return 0;
    return layout(n, capacity, gsi::tiles_x(width) * gsi::tiles_y(height)).bytes;
}

namespace {

// Both entry points: every launch after the counting is sized by the capacity and reads
// the entry count on the device, so nothing here waits for the device.
gs_status bin_sort_launch(const gs_projected *proj, int64_t n, const gs_camera *cam, const gs_raster_params *p,
                          gs_bins *bins, int64_t *counts, void *workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    const float log2_amin = std::log2(p->alpha_min);
    if (!proj || !bins) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    if (n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
    if (n > (int64_t(1) << 31) - 2) return fail(GS_ERR_UNSUPPORTED, "n >= 2^31 - 1");
    if (bins->capacity < 0 || bins->capacity > 0x3FFFFFFFll)
        return fail(GS_ERR_INVALID_ARGUMENT, "capacity out of range (at most 2^30 entries)");
    if (!bins->tile_ranges || (bins->capacity > 0 && !bins->ids))
        return fail(GS_ERR_INVALID_ARGUMENT, "ids / tile_ranges is NULL");
    if (!bins->raster || !aligned(bins->raster, 256))
        return fail(GS_ERR_INVALID_ARGUMENT, "raster buffer is NULL or not 256-byte aligned");
    if (counts && !aligned(counts, 8)) return fail(GS_ERR_INVALID_ARGUMENT, "counts must be 8-byte aligned");
    const int tx = tiles_x(cam->width), ty = tiles_y(cam->height);
    const int32_t T = tx * ty;
    const int64_t cap = bins->capacity;
    const gsr::RasterLayout RL = gsr::raster_layout(n, cap, T);
    char *rb = static_cast<char *>(bins->raster);
    gsr::BinsHeader *hdr = reinterpret_cast<gsr::BinsHeader *>(rb + RL.hdr);
    int32_t *order = reinterpret_cast<int32_t *>(rb + RL.order);
    const int64_t waves = (int64_t)gsr::kQuads * T;
    uint32_t *qoff = reinterpret_cast<uint32_t *>(rb + RL.qoff);
    // the quadrant prefix counts of empty lists: zero
    uint32_t *wpre0 = reinterpret_cast<uint32_t *>(rb + RL.wpre);
    const int64_t nw0 = gsr::kQuads * (RL.words + 1);
    if (n == 0) {
        if ((s = fill_i32(bins->tile_ranges, (int64_t)T + 1, 0, stream)) != GS_OK) return s;
        if ((s = fill_i32(reinterpret_cast<int32_t *>(wpre0), nw0, 0, stream)) != GS_OK) return s;
        k_wave_identity<<<(unsigned)ceil_div(waves, 256), 256, 0, stream>>>((uint32_t)waves, order);
        GS_LAUNCH_CHECK("k_wave_identity");
        k_bins_empty<<<1, 1, 0, stream>>>(hdr, counts, (unsigned long long)RL.grec);
        GS_LAUNCH_CHECK("k_bins_empty");
        return GS_OK;
    }
    if (!proj->depth || !proj->radii || !proj->rec)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected depth / radii / rec is NULL");
    if (!aligned(proj->radii, 8) || !aligned(proj->rec, 16))
        return fail(GS_ERR_INVALID_ARGUMENT, "radii must be 8-byte, rec 16-byte aligned");
    const Layout L = layout(n, cap, T);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.bytes)
        return fail(GS_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, 256-byte aligned", L.bytes);
    char *ws = static_cast<char *>(workspace);
    uint32_t *dkA = (uint32_t *)(ws + L.dkA), *dkB = (uint32_t *)(ws + L.dkB);
    uint64_t *dvA = (uint64_t *)(ws + L.dvA), *dvB = (uint64_t *)(ws + L.dvB);
    uint32_t *qcnt = (uint32_t *)(ws + L.qcnt), *doff = (uint32_t *)(ws + L.doff);
    unsigned long long *total = (unsigned long long *)(ws + L.total);
    unsigned long long *klen = (unsigned long long *)(ws + L.klen);
    uint32_t *tkA = (uint32_t *)(ws + L.tkA), *tkB = (uint32_t *)(ws + L.tkB);
    uint64_t *tvA = (uint64_t *)(ws + L.tvA), *tvB = (uint64_t *)(ws + L.tvB);
    uint32_t *hist = (uint32_t *)(ws + L.hist), *tickets = (uint32_t *)(ws + L.tickets);
    unsigned long long *stD = (unsigned long long *)(ws + L.stD), *stT = (unsigned long long *)(ws + L.stT);
    unsigned long long *scC = (unsigned long long *)(ws + L.scC), *scQ = (unsigned long long *)(ws + L.scQ);
    unsigned long long *scW = (unsigned long long *)(ws + L.scW);
    const int2 *rr = reinterpret_cast<const int2 *>(proj->radii);
    const float4 *prec = reinterpret_cast<const float4 *>(proj->rec);
    const unsigned gn = (unsigned)ceil_div(n, 256);

    // 1. depth keys, tile and quadrant-record counts in index order; the first gradient
    //    slot of each Gaussian (exclusive scan of its record counts) and the total Q; the
    //    same scan zeroes the stamps of the slots it gives out (those that fit), so no slot
    //    of this sort carries a backward call's stamp before one writes it
    float4 *grec = reinterpret_cast<float4 *>(rb + RL.grec);
    k_keys_count<<<gn, 256, 0, stream>>>(rr, proj->depth, prec, log2_amin, n, tx, ty, dkA, dvA, qcnt,
                                         bins->tiles_touched, (uint32_t *)(ws + L.zero), (int64_t)(L.zero_bytes / 4),
                                         grec);
    GS_LAUNCH_CHECK("k_keys_count");
    uint32_t *qstamp = reinterpret_cast<uint32_t *>(rb + RL.qstamp);
    if ((s = lb_scan_u32(qcnt, qoff, n + 1, scQ, tickets + kTkQcnt, total + 1, stream, qstamp,
                         (int64_t)gsr::kQuadFactor * RL.cap)) != GS_OK)
        return s;

    // 2. Gaussians by depth key (stable, so equal keys stay in index order; the values
    //    carry the tile counts along), and the emit offsets: the exclusive scan of the tile
    //    counts in that order, with the total K
    //    It takes three passes instead of four when the visible depth keys span less than
    //    about 2^24 (decided on the device); the result is then in (dkB, dvB), which
    //    xf[1] != 0 tells the scan and the emit pass
    uint32_t *xf = (uint32_t *)(ws + L.xf);   // zeroed by k_keys_count
    bool in_b = false;
    if ((s = radix_sort_u32_u64(dkA, dvA, dkB, dvB, n, 32, hist, stD, tickets + kTkDepth, &in_b, stream, nullptr,
                                xf)) != GS_OK)
        return s;
    const uint32_t *sel = xf + 1;
    if ((s = lb_scan_hi32(dvA, doff, n, scC, tickets + kTkCnt, total, stream, dvB, sel)) != GS_OK) return s;

    // 3. emit entries in depth order (nothing if the lists do not fit), then a stable sort
    //    of (tile key, emit position) by tile
    const int tbits = L.tbits;
    k_emit<<<gn, 256, 0, stream>>>(dvA, dvB, sel, doff, qoff, grec, log2_amin, n, tx, ty, total, cap,
                                   (unsigned long long)RL.grec, klen, hdr, counts, tkA, tvA);
    GS_LAUNCH_CHECK("k_emit");
    if (cap == 0) {
        if ((s = fill_i32(bins->tile_ranges, (int64_t)T + 1, 0, stream)) != GS_OK) return s;
        if ((s = fill_i32(reinterpret_cast<int32_t *>(wpre0), nw0, 0, stream)) != GS_OK) return s;
        k_wave_identity<<<(unsigned)ceil_div(waves, 256), 256, 0, stream>>>((uint32_t)waves, order);
        GS_LAUNCH_CHECK("k_wave_identity");
        return GS_OK;
    }
    // the last pass also writes the Gaussian of each sorted entry to ids (no pass runs for a
    // capacity of 1; k_finish writes them then)
    const bool ids_in_sort = cap > 1;
    if ((s = radix_sort_u32_u64(tkA, tvA, tkB, tvB, cap, tbits, hist, stT, tickets + kTkTile, &in_b, stream, klen,
                                nullptr, ids_in_sort ? bins->ids : nullptr)) != GS_OK)
        return s;
    const uint32_t *tk = in_b ? tkB : tkA;
    const uint64_t *tv = in_b ? tvB : tvA;

    // 4. ids, per-tile ranges, quadrant bitmaps and their scanned bit counts, the quadrant
    //    record lists; optional 64-bit keys
    const unsigned gk = (unsigned)ceil_div(cap, 256);
    uint64_t *bm = reinterpret_cast<uint64_t *>(rb + RL.bitmap);
    uint32_t *wpre = reinterpret_cast<uint32_t *>(rb + RL.wpre);
    const int64_t nw = gsr::kQuads * (RL.words + 1);
    const int64_t fwords = std::max<int64_t>(RL.words, ceil_div((int64_t)T + 1, 64));
    k_finish<<<(unsigned)ceil_div(fwords, 4 * kWaveWords), 256, 0, stream>>>(tk, ids_in_sort ? nullptr : tv, klen, T,
                                                                            bins->ids,
                                                                            bins->tile_ranges, RL.words, bm, wpre);
    GS_LAUNCH_CHECK("k_finish");
    if ((s = lb_scan_u32(wpre, wpre, nw, scW, tickets + kTkWpre, nullptr, stream)) != GS_OK) return s;
    k_quad_lists<<<(unsigned)ceil_div(cap, 4 * 64 * kWaveWords), 256, 0, stream>>>(
        tk, tv, klen, RL.words, wpre, reinterpret_cast<uint2 *>(rb + RL.qent), reinterpret_cast<uint32_t *>(rb + RL.qk));
    GS_LAUNCH_CHECK("k_quad_lists");
    if (bins->keys) {
        k_keys64<<<gk, 256, 0, stream>>>(tk, bins->ids, proj->depth, klen, bins->keys);
        GS_LAUNCH_CHECK("k_keys64");
    }

    // 5. the order in which the (tile, quadrant) waves are rasterized
    {
        uint32_t *whist = (uint32_t *)(ws + L.whist), *wcur = whist + kWaveBuckets;
        uint8_t *wb = (uint8_t *)(ws + L.wb);
        const unsigned gw = (unsigned)ceil_div(waves, 256);
        k_wave_hist<<<gw, 256, 0, stream>>>(bins->tile_ranges, bm, wpre, RL.words, (uint32_t)waves, wb, whist);
        GS_LAUNCH_CHECK("k_wave_hist");
        k_wave_place<<<gw, 256, 0, stream>>>(wb, (uint32_t)waves, whist, wcur, order);
        GS_LAUNCH_CHECK("k_wave_place");
    }
    return GS_OK;
}

}  // namespace

extern "C" gs_status gs_bin_sort_async(const gs_projected *proj, int64_t n, const gs_camera *cam,
                                       const gs_raster_params *p, gs_bins *bins, int64_t *counts, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream)
{
    return bin_sort_launch(proj, n, cam, p, bins, counts, workspace, workspace_bytes, stream);
}

extern "C" gs_status gs_bin_sort(const gs_projected *proj, int64_t n, const gs_camera *cam, const gs_raster_params *p,
                                 gs_bins *bins, int64_t *n_isect_out, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream)
{
    using namespace gsi;
    if (!n_isect_out) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    *n_isect_out = 0;
    gs_status s = bin_sort_launch(proj, n, cam, p, bins, nullptr, workspace, workspace_bytes, stream);
    if (s != GS_OK) return s;
    const gsr::RasterLayout RL =
        gsr::raster_layout(n, bins->capacity, tiles_x(cam->width) * tiles_y(cam->height));
    gsr::BinsHeader h{};
    GS_HIP(hipMemcpyAsync(&h, static_cast<char *>(bins->raster) + RL.hdr, sizeof(h), hipMemcpyDeviceToHost, stream));
    GS_HIP(hipStreamSynchronize(stream));
    *n_isect_out = (int64_t)h.K;
    if (!h.ok) {
        const unsigned long long need = need_capacity(h.K, h.Q);
        *n_isect_out = (int64_t)need;
        return fail(GS_ERR_CAPACITY, "%llu intersections (%llu quadrant records) need a capacity of %llu, have %lld",
                    h.K, h.Q, need, (long long)bins->capacity);
    }
    return GS_OK;
}
