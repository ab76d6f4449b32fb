// Device-wide exclusive scan and stable LSD radix sort for gfx950.
//
// Radix pass (8-bit digit, reduce-then-scan, stable):
//   hist    : each 256-thread block counts the digits of its 2048-element tile
//             (per-wave LDS histograms, one add per run of equal digits across the
//             lanes) and writes them digit-major, so that one
//             exclusive scan over [digit][block] gives every (digit, block) its
//             global output offset;
//   scan    : the single-launch look-back scan below;
//   scatter : each wave ranks its 512 consecutive elements round by round with a
//             64-lane digit match (8 ballots), giving a stable rank per digit; the
//             block then places its tile in LDS in sorted order and writes it out in
//             runs of equal digits (coalesced).
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;
constexpr int kTile = kThreads * kItems;      // 4096 elements per scan block
// radix blocks take 2048 elements, so that a million keys make ~500 blocks and each CU
// holds two or more of them: the ranking loop is latency-bound
constexpr int kRxItems = 8;
constexpr int kRxTile = kThreads * kRxItems;
constexpr int kRxWaveSpan = 64 * kRxItems;

// Exclusive scan of one value per thread across a 256-thread block.  `scratch`
// holds 4 words.  Returns the exclusive prefix; *block_total receives the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch, uint32_t *block_total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) scratch[w] = x;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t s = scratch[k];
        if (k < w) pre += s;
        tot += s;
    }
    __syncthreads();
    *block_total = tot;
    return pre + x - v;
}

__global__ __launch_bounds__(kThreads) void k_scan_reduce(const uint32_t *__restrict__ in, int64_t m,
                                                          uint32_t *__restrict__ partials)
{
    __shared__ uint32_t scratch[4];
    const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
    uint32_t s = 0;
    if (base + kItems <= m) {
        const uint4 *p = reinterpret_cast<const uint4 *>(in + base);
#pragma unroll
        for (int k = 0; k < kItems / 4; ++k) {
            const uint4 q = p[k];
            s += q.x + q.y + q.z + q.w;
        }
    } else {
        for (int k = 0; k < kItems; ++k)
            if (base + k < m) s += in[base + k];
    }
    uint32_t tot;
    block_exclusive_scan(s, scratch, &tot);
    if (threadIdx.x == 0) partials[blockIdx.x] = tot;
}

// Single block: exclusive scan of the block partials, carrying across chunks.
__global__ __launch_bounds__(kThreads) void k_scan_partials(uint32_t *__restrict__ partials, int64_t nb,
                                                            unsigned long long *__restrict__ total)
{
    __shared__ uint32_t scratch[4];
    unsigned long long carry = 0;
    for (int64_t c = 0; c < nb; c += kThreads) {
        const int64_t i = c + threadIdx.x;
        const uint32_t v = i < nb ? partials[i] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(v, scratch, &tot);
        if (i < nb) partials[i] = (uint32_t)(carry + ex);
        carry += tot;
    }
    if (threadIdx.x == 0 && total) *total = carry;
}

__global__ __launch_bounds__(kThreads) void k_scan_down(const uint32_t *__restrict__ in, uint32_t *__restrict__ out,
                                                        int64_t m, const uint32_t *__restrict__ partials)
{
    __shared__ uint32_t scratch[4];
    const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
    uint32_t v[kItems];
    const bool full = base + kItems <= m;
    if (full) {
        const uint4 *p = reinterpret_cast<const uint4 *>(in + base);
#pragma unroll
        for (int k = 0; k < kItems / 4; ++k) {
            const uint4 q = p[k];
            v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kItems; ++k) v[k] = base + k < m ? in[base + k] : 0u;
    }
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < kItems; ++k) s += v[k];
    uint32_t tot;
    uint32_t run = block_exclusive_scan(s, scratch, &tot) + partials[blockIdx.x];
    if (full) {
        uint4 *p = reinterpret_cast<uint4 *>(out + base);
#pragma unroll
        for (int k = 0; k < kItems / 4; ++k) {
            uint4 q;
            q.x = run; run += v[4 * k];
            q.y = run; run += v[4 * k + 1];
            q.z = run; run += v[4 * k + 2];
            q.w = run; run += v[4 * k + 3];
            p[k] = q;
        }
    } else {
        for (int k = 0; k < kItems; ++k)
            if (base + k < m) { out[base + k] = run; run += v[k]; }
    }
}

// m_dev (may be NULL): the element count in device memory, at most m (the launch bound).
__device__ __forceinline__ int64_t elem_count(int64_t m, const unsigned long long *m_dev)
{
    return m_dev ? (int64_t)min((unsigned long long)m, *m_dev) : m;
}

// Key range reduction of a 32-bit sort.  xf: kRadixXfWords device words, zero before the
// sort.  The first pass's histogram also gathers the largest key and the largest
// complement of a key over the keys other than 0xFFFFFFFF, each block into one of kXfSlots
// slots (one 128-byte line each, so that the blocks' atomics spread over the memory
// channels); from them the first scatter derives the offset o (the smallest key with its
// low byte cleared) and whether every such key k has k - o < 0xFFFFFF, and stores both in
// xf[0], xf[1].  If it does, that scatter writes every key k as k - o, and 0xFFFFFFFF (an
// element whose place among the other keys does not matter, as a culled Gaussian's, but
// which sorts last) as 0xFFFFFF: the order is unchanged, the fourth digit is then zero for
// every key, and the fourth pass skips itself.  The first digit is the same before and
// after the change (o's low byte is zero), so the first histogram is taken before o is
// known.  Modes of a pass (a template argument): 0 plain, 1 the first pass, 2 the fourth
// pass.
constexpr int kXfSlots = 32, kXfSlotWords = 32;
static_assert(gsi::kRadixXfWords == kXfSlotWords * (1 + kXfSlots), "xf layout");

__device__ __forceinline__ uint32_t *xf_slot(uint32_t *xf, int s) { return xf + kXfSlotWords * (1 + s); }

// Every lane of the calling wave gets o and fits (lanes 0 .. kXfSlots - 1 read one slot each).
__device__ __forceinline__ void xf_range(uint32_t *xf, uint32_t &o, bool &fits)
{
    const int lane = threadIdx.x & 63;
    uint32_t mx = 0u, ninv = 0u;
    if (lane < kXfSlots) {
        const uint32_t *sl = xf_slot(xf, lane);
        mx = sl[0];
        ninv = sl[1];
    }
    for (int d = 32; d > 0; d >>= 1) {   // over all 64 lanes: every lane needs the result
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
        ninv = max(ninv, (uint32_t)__shfl_xor((int)ninv, d, 64));
    }
    o = ninv ? ~ninv & ~0xFFu : 0u;   // ninv == 0: no key other than 0xFFFFFFFF
    fits = ninv == 0u || mx - o < 0xFFFFFFu;
}

template <int MODE>
__device__ __forceinline__ bool xf_skip(const uint32_t *__restrict__ xf)
{
    return MODE == 2 && xf[1] != 0u;
}

// The radix tile a block takes.  Blocks reach the 8 XCDs round-robin (block b on XCD
// b % 8); the tiles that hold elements are renumbered so that each XCD takes one
// contiguous run of them.  Neighbouring tiles write neighbouring words of the digit-major
// histogram and neighbouring runs of each digit's output, so their partial cache lines
// meet in one L2 instead of eight.  Tiles past the last element keep their own number.
__device__ __forceinline__ int64_t rx_tile(int64_t m)
{
    const int64_t b = blockIdx.x, active = (m + kRxTile - 1) / kRxTile;
    if (b >= active) return b;
    const int64_t x = b % gsi::kXcds, per = active / gsi::kXcds, rem = active % gsi::kXcds;
    return x * per + (x < rem ? x : rem) + b / gsi::kXcds;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_radix_hist(const uint32_t *__restrict__ keys, int64_t m_max,
                                                         const unsigned long long *__restrict__ m_dev, int shift,
                                                         uint32_t *__restrict__ hist, int64_t nb,
                                                         uint32_t *__restrict__ xf)
{
    __shared__ uint32_t h[4][256];
    __shared__ uint32_t red[2][4];
    if (xf_skip<MODE>(xf)) return;   // the whole grid
    const int64_t m = elem_count(m_max, m_dev);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t tile = rx_tile(m);
    for (int i = threadIdx.x; i < 4 * 256; i += kThreads) (&h[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = tile * kRxTile + (int64_t)w * kRxWaveSpan + lane;
    // Consecutive lanes hold consecutive elements.  Each run of equal digits across the
    // lanes is counted by its first lane with one LDS add of the run length, so skewed or
    // presorted keys (long runs of one digit) do not serialise on one LDS address.
    uint32_t kmax = 0u, kninv = 0u;   // over the keys other than 0xFFFFFFFF (MODE 1)
#pragma unroll 4
    for (int r = 0; r < kRxItems; ++r) {
        const int64_t e = base + r * 64;
        const bool valid = e < m;
        const uint32_t kv = valid ? keys[e] : 0xFFFFFFFFu;
        if (MODE == 1 && kv != 0xFFFFFFFFu) {
            kmax = max(kmax, kv);
            kninv = max(kninv, ~kv);
        }
        const uint32_t d = valid ? (kv >> shift) & 255u : 0x100u;   // 0x100: no element
        const uint32_t dp = __shfl_up(d, 1, 64);
        const bool head = lane == 0 || d != dp;
        const uint64_t heads = __ballot(head);
        if (head && valid) {
            const uint64_t above = lane == 63 ? 0ull : heads >> (lane + 1);
            const int next = above ? lane + 1 + __builtin_ctzll(above) : 64;
            atomicAdd(&h[w][d], (uint32_t)(next - lane));
        }
    }
    if (MODE == 1) {
        for (int o = 32; o > 0; o >>= 1) {
            kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
            kninv = max(kninv, (uint32_t)__shfl_xor((int)kninv, o, 64));
        }
        if (lane == 0) {
            red[0][w] = kmax;
            red[1][w] = kninv;
        }
    }
    __syncthreads();
    const int d = threadIdx.x;
    hist[(int64_t)d * nb + tile] = h[0][d] + h[1][d] + h[2][d] + h[3][d];
    if (MODE == 1 && threadIdx.x < 2) {
        const uint32_t *r4 = red[threadIdx.x];
        const uint32_t v = max(max(r4[0], r4[1]), max(r4[2], r4[3]));
        if (v) atomicMax(xf_slot(xf, (int)(blockIdx.x % kXfSlots)) + threadIdx.x, v);
    }
}

template <typename V, int MODE>
__global__ __launch_bounds__(kThreads) void k_radix_scatter(const uint32_t *__restrict__ kin, const V *__restrict__ vin,
                                                            uint32_t *__restrict__ kout, V *__restrict__ vout,
                                                            int64_t m_max, const unsigned long long *__restrict__ m_dev,
                                                            int shift, const uint32_t *__restrict__ offs, int64_t nb,
                                                            uint32_t *__restrict__ xf, uint32_t *__restrict__ low_out)
{
    if (xf_skip<MODE>(xf)) return;   // the whole grid
    uint32_t xo = 0u;
    bool tf = false;
    if (MODE == 1) {
        xf_range(xf, xo, tf);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            xf[0] = xo;
            xf[1] = tf ? 1u : 0u;
        }
    }
    const int64_t m = elem_count(m_max, m_dev);
    __shared__ uint32_t wcnt[4][256];
    __shared__ uint32_t bstart[256];
    __shared__ uint32_t gbase[256];
    __shared__ uint32_t scratch[4];
    __shared__ uint32_t skey[kRxTile];
    __shared__ V sval[kRxTile];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t tile = rx_tile(m), tile0 = tile * kRxTile;
    if (tile0 >= m) return;   // the whole block: nothing to place
    for (int i = threadIdx.x; i < 4 * 256; i += kThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = tile0 + (int64_t)w * kRxWaveSpan + lane;
    const uint64_t below_mask = (1ull << lane) - 1ull;
    uint32_t key[kRxItems], rank[kRxItems];
    V val[kRxItems];
#pragma unroll
    for (int r = 0; r < kRxItems; ++r) {
        const int64_t e = base + r * 64;
        const bool valid = e < m;
        uint32_t k = valid ? kin[e] : 0u;
        if (tf) k = k == 0xFFFFFFFFu ? 0xFFFFFFu : k - xo;
        const V v = valid ? vin[e] : V(0);
        const uint32_t d = (k >> shift) & 255u;
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            same &= bit ? bb : ~bb;
        }
        const uint32_t below = (uint32_t)__popcll(same & below_mask);
        const uint32_t cnt = (uint32_t)__popcll(same);
        const uint32_t prev = wcnt[w][d];
        __builtin_amdgcn_wave_barrier();
        if (valid && below == 0) wcnt[w][d] = prev + cnt;
        __builtin_amdgcn_wave_barrier();
        key[r] = k;
        val[r] = v;
        rank[r] = prev + below;
    }
    __syncthreads();
    {
        const int d = threadIdx.x;
        const uint32_t c0 = wcnt[0][d], c1 = wcnt[1][d], c2 = wcnt[2][d], c3 = wcnt[3][d];
        wcnt[0][d] = 0;
        wcnt[1][d] = c0;
        wcnt[2][d] = c0 + c1;
        wcnt[3][d] = c0 + c1 + c2;
        uint32_t tot;
        bstart[d] = block_exclusive_scan(c0 + c1 + c2 + c3, scratch, &tot);
        gbase[d] = offs[(int64_t)d * nb + tile];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRxItems; ++r) {
        const int64_t e = base + r * 64;
        if (e < m) {
            const uint32_t d = (key[r] >> shift) & 255u;
            const uint32_t p = bstart[d] + wcnt[w][d] + rank[r];
            skey[p] = key[r];
            sval[p] = val[r];
        }
    }
    __syncthreads();
    const int cnt = (int)min((int64_t)kRxTile, m - tile0);
    for (int i = threadIdx.x; i < cnt; i += kThreads) {
        const uint32_t k = skey[i];
        const uint32_t d = (k >> shift) & 255u;
        const uint32_t dst = gbase[d] + ((uint32_t)i - bstart[d]);
        if (dst < (uint64_t)m) {   // always true for a consistent ranking; keeps a bug from writing out of bounds
            kout[dst] = k;
            vout[dst] = sval[i];
            if (low_out) low_out[dst] = (uint32_t)sval[i];
        }
    }
}

// ------------------------------------------------------------------ single-launch scan
//
// Each block takes the next tile of values in arrival order (an atomic ticket: any
// tile it waits for belongs to a block that has already started), publishes its sum, and
// finds the sum of everything before it by looking back over the published sums, 64 tiles
// per step (one wave, one status word per lane), until it meets a tile that has published
// its inclusive prefix.  In the steady state each tile waits for its predecessor's
// inclusive prefix, a chain of ~45 ns per tile on MI355X (measured; wider windows of 8
// words per lane were slower), so large scans take larger tiles: 4096 values up to 1.5M,
// 8192 up to 6M, 16384 above (the chain, not the bandwidth, bounds a scan of 10M values
// with 4096-value tiles).  64-bit status words: flag in bits 62..63 (0 = not yet published,
// 1 = the tile's own sum, 2 = its inclusive prefix), the sum below.
constexpr unsigned long long kFlagSum = 1ull << 62, kFlagIncl = 2ull << 62, kFlagMask = 3ull << 62;

__device__ __forceinline__ unsigned long long status_load(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void status_store(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Tile size of the single-launch scan for m values: kThreads * lb_items(m) values.
__host__ __device__ constexpr int lb_items(int64_t m) { return m <= 1500000 ? 16 : m <= 6000000 ? 32 : 64; }

// HI32: the input is uint64 and the scan takes the high 32 bits of each value.
// clear (nullable): the tile also sets clear[x] = 0 for x in its own output range
// [prefix, prefix + tile sum) below clear_lim, so that one coalesced pass zeroes the
// elements the scanned counts give out (each tile's range is contiguous).
// DEV only: skip (nullable): when *skip != 0 the whole scan does nothing (no block takes a
// ticket); in_alt, sel (nullable): when *sel != 0 the input is in_alt instead of in_v.
template <int ITEMS, bool HI32, bool DEV>
__global__ __launch_bounds__(kThreads) void k_scan_lb(const void *in_v, uint32_t *out, int64_t m,
                                                      unsigned long long *__restrict__ status,
                                                      uint32_t *__restrict__ ticket,
                                                      unsigned long long *__restrict__ total,
                                                      uint32_t *__restrict__ clear, int64_t clear_lim,
                                                      const uint32_t *__restrict__ skip, const void *in_alt,
                                                      const uint32_t *__restrict__ sel)
{
    constexpr int kT = kThreads * ITEMS;
    __shared__ uint32_t scratch[4];
    __shared__ uint32_t s_tile;
    __shared__ unsigned long long s_excl;
    if (DEV) {
        if (skip && *skip) return;   // uniform over the grid
        if (sel && *sel) in_v = in_alt;
    }
    if (threadIdx.x == 0) s_tile = atomicAdd(ticket, 1u);
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t base = tile * kT + (int64_t)threadIdx.x * ITEMS;
    uint32_t v[ITEMS];
    const bool full = base + ITEMS <= m;
    if (HI32) {
        const uint64_t *in = static_cast<const uint64_t *>(in_v);
        if (full) {
            const ulonglong2 *p = reinterpret_cast<const ulonglong2 *>(in + base);
#pragma unroll
            for (int k = 0; k < ITEMS / 2; ++k) {
                const ulonglong2 q = p[k];
                v[2 * k] = (uint32_t)(q.x >> 32); v[2 * k + 1] = (uint32_t)(q.y >> 32);
            }
        } else {
#pragma unroll
            for (int k = 0; k < ITEMS; ++k) v[k] = base + k < m ? (uint32_t)(in[base + k] >> 32) : 0u;
        }
    } else {
        const uint32_t *in = static_cast<const uint32_t *>(in_v);
        if (full) {
            const uint4 *p = reinterpret_cast<const uint4 *>(in + base);
#pragma unroll
            for (int k = 0; k < ITEMS / 4; ++k) {
                const uint4 q = p[k];
                v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < ITEMS; ++k) v[k] = base + k < m ? in[base + k] : 0u;
        }
    }
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) sum += v[k];
    uint32_t tot32;
    const uint32_t pre = block_exclusive_scan(sum, scratch, &tot32);
    const unsigned long long tot = tot32;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        if (lane == 0) status_store(status + tile, (tile == 0 ? kFlagIncl : kFlagSum) | tot);
        unsigned long long excl = 0;
        if (tile > 0) {
            for (int64_t hi = tile - 1;; hi -= 64) {
                const int64_t j = hi - lane;   // lane 0 is the nearest tile
                // before tile 0 everything is an inclusive prefix of 0
                unsigned long long x = j >= 0 ? status_load(status + j) : kFlagIncl;
                while (__ballot((x & kFlagMask) == 0ull)) {   // wait for the window to be published
                    __builtin_amdgcn_s_sleep(1);
                    if ((x & kFlagMask) == 0ull) x = status_load(status + j);
                }
                const uint64_t incl = __ballot((x & kFlagMask) == kFlagIncl);
                if (incl) {
                    const int first = __ffsll((long long)incl) - 1;   // nearest inclusive prefix
                    excl += wave_sum_u64(lane <= first ? (x & ~kFlagMask) : 0ull);
                    break;
                }
                excl += wave_sum_u64(x & ~kFlagMask);
            }
        }
        if (lane == 0) {
            if (tile > 0) status_store(status + tile, kFlagIncl | (excl + tot));
            s_excl = excl;
            if (total && (tile + 1) * kT >= m) *total = excl + tot;   // the last tile
        }
    }
    __syncthreads();
    if (clear) {
        const int64_t c0 = (int64_t)s_excl, c1 = min((int64_t)(s_excl + tot), clear_lim);
        for (int64_t x = c0 + threadIdx.x; x < c1; x += kThreads) clear[x] = 0u;
    }
    uint32_t run = (uint32_t)s_excl + pre;
    if (full) {
        uint4 *p = reinterpret_cast<uint4 *>(out + base);
#pragma unroll
        for (int k = 0; k < ITEMS / 4; ++k) {
            uint4 q;
            q.x = run; run += v[4 * k];
            q.y = run; run += v[4 * k + 1];
            q.z = run; run += v[4 * k + 2];
            q.w = run; run += v[4 * k + 3];
            p[k] = q;
        }
    } else {
        for (int k = 0; k < ITEMS; ++k)
            if (base + k < m) { out[base + k] = run; run += v[k]; }
    }
}

template <bool HI32>
gs_status launch_scan_lb(const void *in, uint32_t *out, int64_t m, unsigned long long *status, uint32_t *ticket,
                         unsigned long long *total, hipStream_t stream, uint32_t *clear = nullptr,
                         int64_t clear_lim = 0, const uint32_t *skip = nullptr, const void *in_alt = nullptr,
                         const uint32_t *sel = nullptr)
{
    if (m <= 0) return gsi::fail(GS_ERR_UNSUPPORTED, "scan of an empty array");
    const int items = lb_items(m);
    const unsigned grid = (unsigned)gsi::ceil_div(m, (int64_t)kThreads * items);
    const bool dev = skip || sel;
#define GS_SCAN_LB(IT, D)                                                                                           \
    k_scan_lb<IT, HI32, D><<<grid, kThreads, 0, stream>>>(in, out, m, status, ticket, total, clear, clear_lim, skip, \
                                                          in_alt, sel)
    if (items == 16) {
        if (dev) GS_SCAN_LB(16, true); else GS_SCAN_LB(16, false);
    } else if (items == 32) {
        if (dev) GS_SCAN_LB(32, true); else GS_SCAN_LB(32, false);
    } else {
        if (dev) GS_SCAN_LB(64, true); else GS_SCAN_LB(64, false);
    }
#undef GS_SCAN_LB
    GS_LAUNCH_CHECK("k_scan_lb");
    return GS_OK;
}

__global__ void k_fill_i32(int32_t *__restrict__ p, int64_t n, int32_t value)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

__global__ void k_fill_f32(float *__restrict__ p, int64_t n, float value)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

}  // namespace

namespace gsi {

int64_t scan_partials_len(int64_t m) { return ceil_div(m > 0 ? m : 1, kTile); }

gs_status exclusive_scan_u32(const uint32_t *in, uint32_t *out, int64_t m, uint32_t *partials,
                             unsigned long long *total, hipStream_t stream)
{
    if (m <= 0) {
        if (total) {   // a kernel, not a memset: keeps the call capturable in a graph
            k_scan_partials<<<1, kThreads, 0, stream>>>(partials, 0, total);
            GS_LAUNCH_CHECK("k_scan_partials");
        }
        return GS_OK;
    }
    const int64_t nb = scan_partials_len(m);
    if (nb > 0x7fffffff) return fail(GS_ERR_UNSUPPORTED, "scan too large");
    k_scan_reduce<<<(unsigned)nb, kThreads, 0, stream>>>(in, m, partials);
    GS_LAUNCH_CHECK("k_scan_reduce");
    k_scan_partials<<<1, kThreads, 0, stream>>>(partials, nb, total);
    GS_LAUNCH_CHECK("k_scan_partials");
    k_scan_down<<<(unsigned)nb, kThreads, 0, stream>>>(in, out, m, partials);
    GS_LAUNCH_CHECK("k_scan_down");
    return GS_OK;
}

int64_t radix_hist_len(int64_t m) { return 256 * ceil_div(m > 0 ? m : 1, kRxTile); }

int64_t lb_scan_tiles(int64_t m) { return ceil_div(m > 0 ? m : 1, (int64_t)kThreads * lb_items(m)); }

gs_status lb_scan_u32(const uint32_t *in, uint32_t *out, int64_t m, unsigned long long *status, uint32_t *ticket,
                      unsigned long long *total, hipStream_t stream, uint32_t *clear, int64_t clear_lim)
{
    return launch_scan_lb<false>(in, out, m, status, ticket, total, stream, clear, clear_lim);
}

gs_status lb_scan_hi32(const uint64_t *in, uint32_t *out, int64_t m, unsigned long long *status, uint32_t *ticket,
                       unsigned long long *total, hipStream_t stream, const uint64_t *in_alt, const uint32_t *sel)
{
    if (!aligned(in, 16) || (in_alt && !aligned(in_alt, 16)))
        return fail(GS_ERR_INVALID_ARGUMENT, "scan input must be 16-byte aligned");
    return launch_scan_lb<true>(in, out, m, status, ticket, total, stream, nullptr, 0, nullptr, in_alt, sel);
}

int64_t radix_scan_status_len(int64_t m, int bits)
{
    return (int64_t)((bits + 7) / 8) * lb_scan_tiles(radix_hist_len(m));
}

template <typename V>
gs_status radix_sort_kv(uint32_t *ka, V *va, uint32_t *kb, V *vb, int64_t m, int bits, uint32_t *hist,
                        unsigned long long *scan_status, uint32_t *scan_tickets, bool *in_b, hipStream_t stream,
                        const unsigned long long *m_dev, uint32_t *xf, uint32_t *low_out)
{
    if (xf && bits != 32) return fail(GS_ERR_INVALID_ARGUMENT, "key range reduction needs a 32-bit sort");
    if (xf && low_out) return fail(GS_ERR_INVALID_ARGUMENT, "low_out with key range reduction");
    *in_b = false;
    if (m <= 1 || bits <= 0) return GS_OK;
    const int64_t nb = ceil_div(m, kRxTile);
    const int passes = (bits + 7) / 8;
    uint32_t *sk = ka, *dk = kb;
    V *sv = va, *dv = vb;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        const int mode = !xf ? 0 : p == 0 ? 1 : p == 3 ? 2 : 0;
        uint32_t *lo = p == passes - 1 ? low_out : nullptr;
        if (mode == 1)
            k_radix_hist<1><<<(unsigned)nb, kThreads, 0, stream>>>(sk, m, m_dev, shift, hist, nb, xf);
        else if (mode == 2)
            k_radix_hist<2><<<(unsigned)nb, kThreads, 0, stream>>>(sk, m, m_dev, shift, hist, nb, xf);
        else
            k_radix_hist<0><<<(unsigned)nb, kThreads, 0, stream>>>(sk, m, m_dev, shift, hist, nb, xf);
        GS_LAUNCH_CHECK("k_radix_hist");
        gs_status s = launch_scan_lb<false>(hist, hist, 256 * nb, scan_status + p * lb_scan_tiles(256 * nb),
                                            scan_tickets + p, nullptr, stream, nullptr, 0,
                                            mode == 2 ? xf + 1 : nullptr);
        if (s != GS_OK) return s;
        if (mode == 1)
            k_radix_scatter<V, 1><<<(unsigned)nb, kThreads, 0, stream>>>(sk, sv, dk, dv, m, m_dev, shift, hist, nb, xf,
                                                                         lo);
        else if (mode == 2)
            k_radix_scatter<V, 2><<<(unsigned)nb, kThreads, 0, stream>>>(sk, sv, dk, dv, m, m_dev, shift, hist, nb, xf,
                                                                         lo);
        else
            k_radix_scatter<V, 0><<<(unsigned)nb, kThreads, 0, stream>>>(sk, sv, dk, dv, m, m_dev, shift, hist, nb, xf,
                                                                         lo);
        GS_LAUNCH_CHECK("k_radix_scatter");
        std::swap(sk, dk);
        std::swap(sv, dv);
        *in_b = !*in_b;
    }
    return GS_OK;
}

gs_status radix_sort_u32(uint32_t *ka, uint32_t *va, uint32_t *kb, uint32_t *vb, int64_t m, int bits,
                         uint32_t *hist, unsigned long long *scan_status, uint32_t *scan_tickets, bool *in_b,
                         hipStream_t stream, const unsigned long long *m_dev)
{
    return radix_sort_kv(ka, va, kb, vb, m, bits, hist, scan_status, scan_tickets, in_b, stream, m_dev, nullptr,
                         nullptr);
}

gs_status radix_sort_u32_u64(uint32_t *ka, uint64_t *va, uint32_t *kb, uint64_t *vb, int64_t m, int bits,
                             uint32_t *hist, unsigned long long *scan_status, uint32_t *scan_tickets, bool *in_b,
                             hipStream_t stream, const unsigned long long *m_dev, uint32_t *xf, uint32_t *low_out)
{
    return radix_sort_kv(ka, va, kb, vb, m, bits, hist, scan_status, scan_tickets, in_b, stream, m_dev, xf, low_out);
}

gs_status fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t stream)
{
    if (n <= 0) return GS_OK;
    k_fill_i32<<<(unsigned)ceil_div(n, 256), 256, 0, stream>>>(p, n, value);
    GS_LAUNCH_CHECK("k_fill_i32");
    return GS_OK;
}

gs_status fill_f32(float *p, int64_t n, float value, hipStream_t stream)
{
    if (n <= 0) return GS_OK;
    k_fill_f32<<<(unsigned)ceil_div(n, 256), 256, 0, stream>>>(p, n, value);
    GS_LAUNCH_CHECK("k_fill_f32");
    return GS_OK;
}

}  // namespace gsi
