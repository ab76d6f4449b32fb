// Per-quadrant record walks shared by the raster kernels (the forward, the backward and the
// fused forward + L1 + backward), so that they evaluate every (pixel, record) pair with the
// same instructions.  One 64-lane wave per 8x8 quadrant of a 16x16 tile, one pixel per lane
// (lane & 7 = column, lane >> 3 = row); records come through scalar loads (raster.h).
#pragma once

#include "raster.h"

namespace gsr {

// The quadrant lists hold per record its Gaussian g and gradient slot (qent); the record
// itself (centre, pre-scaled conic, log2 opacity, colour) is the Gaussian's raster record
// in grec, fetched by g with scalar loads.  A wave reads the entries of its list 64
// at a time with one vector load (lane l: entry c + l), two chunks ahead, and takes each
// record's g and slot out of those registers (v_readlane).  One chunk ahead, each lane
// also loads one word of its entry's record, so that the records a chunk's scalar loads
// fetch are in L2 by then (the records are scattered over the Gaussian array; without it
// each batch waited for HBM).
struct Chunks {
    uint2 e0, e1, e2;   // entries of chunks base, base + 64 and base + 128
    float pf;           // the record word loaded to warm L2 (consumed one chunk later)
    uint32_t base, last;
    const uint2 *qent;
    const float4 *grec;
    // Lane l loads entry c + l, clamped to the list's last entry: the loads are unconditional
    // (no divergent branch, so the compiler's waits on them stay exact), and a lane past the
    // list names a real Gaussian, whose record is loaded and never used.
    __device__ __forceinline__ uint2 load(uint32_t c) const { return qent[min(c + (uint32_t)threadIdx.x, last)]; }
    // e0 is always written by an explicit move (of a loaded value that has arrived), never
    // straight by a load: the compiler's wait placement then knows that reading e0 needs no
    // wait, also where vector stores are in flight (they share the load counter on this GPU).
    __device__ __forceinline__ static uint2 moved(uint2 v)
    {
        uint32_t x, y;
        asm volatile("v_mov_b32 %0, %2\n\tv_mov_b32 %1, %3" : "=v"(x), "=v"(y) : "v"(v.x), "v"(v.y));
        return make_uint2(x, y);
    }
    // one word of the record of this lane's entry of chunk base + 64 (e1, arrived)
    __device__ __forceinline__ void warm() { pf = grec[kGRecF4 * (size_t)e1.x].x; }
    // for a non-empty list j0 .. j1
    __device__ __forceinline__ void init(const uint2 *q, const float4 *g, uint32_t j0, uint32_t j1)
    {
        qent = q;
        grec = g;
        base = j0;
        last = j1 - 1u;
        const uint2 first = load(j0);
        const uint2 second = load(j0 + 64u);
        e0 = moved(first);
        e1 = moved(second);
        __builtin_amdgcn_sched_barrier(0);
        warm();
        e2 = load(j0 + 128u);
    }
    // at the first record of the next chunk (its entries were loaded two chunks ago, those
    // of the chunk after it one chunk ago).  The moves are ordered before the next loads, so
    // that the loads can write their registers directly: as plain assignments, the compiler
    // issued the loads into temporaries and copied them afterwards, which waits for the
    // loads just issued.
    __device__ __forceinline__ void advance()
    {
        base += 64u;
        asm volatile("" ::"v"(pf));   // the previous warming load (long arrived)
        e0 = moved(e1);
        e1 = moved(e2);
        __builtin_amdgcn_sched_barrier(0);
        warm();
        e2 = load(base + 128u);
    }
    // entries of records j .. j + kN - 1 (all in one chunk: base <= j, j + kN <= base + 128,
    // j - base a multiple of kN), uniform across the wave; the chunk is chosen by a uniform
    // branch, so a batch reads only its own chunk's registers
    template <int kN>
    __device__ __forceinline__ void at(uint32_t j, uint32_t (&g)[kN], uint32_t (&slot)[kN]) const
    {
        const uint32_t l = j - base;
        const int ln = (int)(l & 63u);
        if (l < 64u) {
#pragma unroll
            for (int i = 0; i < kN; ++i) {
                g[i] = (uint32_t)__builtin_amdgcn_readlane((int)e0.x, ln + i);
                slot[i] = (uint32_t)__builtin_amdgcn_readlane((int)e0.y, ln + i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kN; ++i) {
                g[i] = (uint32_t)__builtin_amdgcn_readlane((int)e1.x, ln + i);
                slot[i] = (uint32_t)__builtin_amdgcn_readlane((int)e1.y, ln + i);
            }
        }
    }
    template <int kN>
    __device__ __forceinline__ void at(uint32_t j, uint32_t (&g)[kN]) const
    {
        const uint32_t l = j - base;
        const int ln = (int)(l & 63u);
        if (l < 64u) {
#pragma unroll
            for (int i = 0; i < kN; ++i) g[i] = (uint32_t)__builtin_amdgcn_readlane((int)e0.x, ln + i);
        } else {
#pragma unroll
            for (int i = 0; i < kN; ++i) g[i] = (uint32_t)__builtin_amdgcn_readlane((int)e1.x, ln + i);
        }
    }
    __device__ __forceinline__ void finish() const { asm volatile("" ::"v"(pf)); }
};

// One batch of records in scalar registers.
template <int kFwdBatch>
struct Batch {
    float4 p0[kFwdBatch], p1[kFwdBatch];
    float blue[kFwdBatch];
    // records j .. j + kFwdBatch - 1 of the list (entries past its end repeat the last one,
    // loaded and never used)
    __device__ __forceinline__ void load(const Chunks &C, uint32_t j)
    {
        uint32_t g[kFwdBatch];
        C.at<kFwdBatch>(j, g);
#pragma unroll
        for (int i = 0; i < kFwdBatch; ++i) {
            const float4 *rb = C.grec + kGRecF4 * (size_t)g[i];
            p0[i] = rb[0];
            p1[i] = rb[1];
            blue[i] = rb[2].x;
        }
    }
    // Makes the loaded values available here: the compiler waits for the scalar loads at
    // this point (the "memory" clobber keeps later loads behind it).
    __device__ __forceinline__ void wait() const
    {
#pragma unroll
        for (int i = 0; i < kFwdBatch; ++i)
            asm volatile("" ::"s"(p0[i].x), "s"(p0[i].y), "s"(p0[i].z), "s"(p0[i].w), "s"(p1[i].x), "s"(p1[i].y),
                         "s"(p1[i].z), "s"(p1[i].w), "s"(blue[i])
                         : "memory");
    }
};

// ByteSplat Eq. 1 over the quadrant's records j0 .. j1 (tile list entries start .. end):
// front-to-back compositing of the lane's pixel at (fx, fy), stopping once T < t_min.
// Outputs the colour (cr, cg, cb), T_final and N_p (entries of the tile list traversed: the
// tile-list index qk of the record at which the pixel stopped, minus start, plus one; the
// whole list if it never stopped).
// kFwdBatch (2 or 4) records per scalar-load batch, two batches in flight: 4 hides more
// load latency, 2 needs 40 fewer scalar registers (the fused kernel's backward phase then
// keeps more waves resident).  The batch size does not change the arithmetic.
// With kCount, walked receives the number of records the wave evaluated (each for all 64
// lanes) and taken the number of them this lane accepted (alpha-check passed while live);
// without it both are left alone.
template <int kFwdBatch = 4, bool kCount = false>
__device__ __forceinline__ void fwd_walk(const uint2 *__restrict__ qent, const uint32_t *__restrict__ qk,
                                         const float4 *__restrict__ grec, uint32_t j0, uint32_t j1, float fx,
                                         float fy, int start, int end, bool inside, float alpha_min, float alpha_max,
                                         float t_min, float &cr, float &cg, float &cb, float &Tr, int &np,
                                         uint32_t *walked = nullptr, uint32_t *taken = nullptr)
{
    Tr = 1.0f;
    cr = 0.0f;
    cg = 0.0f;
    cb = 0.0f;
    np = end - start;
    uint32_t jstop = 0xFFFFFFFFu;   // the record at which this lane's pixel stopped
    bool live = inside;
    if constexpr (kCount) *walked = 0u;
    if (j0 >= j1) return;   // no record reaches the quadrant: the pixels traverse the whole list
    Chunks C;
    C.init(qent, grec, j0, j1);
    // Records come in batches of kFwdBatch through scalar loads.  Scalar loads complete out
    // of order, so the only wait is for all of them: the loop waits for batch b, issues the
    // loads of batch b + 1 and then blends batch b, so that the loads of b + 1 land while b
    // is blended.  Two register sets, alternating (the loop body is unrolled twice).
    Batch<kFwdBatch> A, B;
    A.load(C, j0);
    auto blend = [&](const Batch<kFwdBatch> &R, uint32_t j) {
        // branch-free per entry: lanes that do not take it blend with alpha = 0 (T and C
        // unchanged exactly); termination is a mask update
#pragma unroll
        for (int i = 0; i < kFwdBatch; ++i) {
            if (j + (uint32_t)i >= j1) break;
            const float dx = fx - R.p0[i].x, dy = fy - R.p0[i].y;
            const float alpha = fminf(alpha_max, exp2_fast(exponent(R.p0[i], R.p1[i], dx, dy)));
            const bool take = live && alpha >= alpha_min;
            if constexpr (kCount) *taken += take ? 1u : 0u;
            const float a = take ? alpha : 0.0f;
            const float w = Tr * a;
            cr = fmaf(w, R.p1[i].z, cr);
            cg = fmaf(w, R.p1[i].w, cg);
            cb = fmaf(w, R.blue[i], cb);
            Tr = Tr * (1.0f - a);
            const bool stop = take && Tr < t_min;
            jstop = stop ? j + (uint32_t)i : jstop;
            live = live && !stop;
        }
    };
    auto chunk = [&](uint32_t j) {
        if (((j - j0) & 63u) == 0u && j > j0) C.advance();
    };
    uint32_t jw = j0;   // end of the records blended so far
    for (uint32_t j = j0; j < j1; j += 2 * kFwdBatch) {
        chunk(j);
        A.wait();
        B.load(C, j + kFwdBatch);   // past j1: the last entry again, loaded but unused
        blend(A, j);
        if constexpr (kCount) jw = min(j + kFwdBatch, j1);
        if (j + kFwdBatch >= j1 || __ballot(live) == 0) break;
        chunk(j + kFwdBatch);
        B.wait();
        A.load(C, j + 2 * kFwdBatch);
        blend(B, j + kFwdBatch);
        if constexpr (kCount) jw = min(j + 2 * kFwdBatch, j1);
        if (__ballot(live) == 0) break;
    }
    C.finish();
    if (jstop != 0xFFFFFFFFu) np = (int)qk[jstop] - start + 1;
    if constexpr (kCount) *walked = jw - j0;
}

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

// ByteSplat Eq. 3 (and the per-record part of Eq. 4) over the quadrant's records j0 .. j1,
// front to back, for the lane's pixel at (fx, fy) with dL/dC = (G0, G1, G2),
// Z = C . G + G_T T_final; the pixel takes records j < jend (jend: the quadrant position of
// the first entry beyond its N_p, quad_prefix(start + N_p)).  The moment sums of every
// batch of 4 records some pixel takes go to the records' gradient slots in qgrad, stamped
// with epoch in qstamp.
__device__ __forceinline__ void bwd_walk(const uint2 *__restrict__ qent, const float4 *__restrict__ grec, uint32_t j0,
                                         uint32_t j1, float fx, float fy, uint32_t jend, float G0, float G1, float G2,
                                         float Z, float alpha_min, float alpha_max, uint32_t epoch,
                                         float *__restrict__ qgrad, uint32_t *__restrict__ qstamp)
{
    const int lane = threadIdx.x & 63;
    const int row = lane >> 4, nl = lane & 15;
    // the reduced field each lane of a row holds (reduce_4x9): even lanes hold fields 0-7,
    // lane 1 field 8; lane 3 writes the slot's stamp (the epoch)
    const bool stamp_lane = nl == 3;
    const int my_field = nl == 1 ? 8 : 4 * ((nl >> 1) & 1) + 2 * ((nl >> 2) & 1) + ((nl >> 3) & 1);
    const bool lane_writes = (nl & 1) == 0 || nl == 1 || stamp_lane;
    float Tr = 1.0f;
    if (j0 >= j1) return;
    Chunks C;
    C.init(qent, grec, j0, j1);
    for (uint32_t jt = j0; jt < j1;) {
        if (((jt - j0) & 63u) == 0u && jt > j0) C.advance();
        // records jt .. jt+3 (past j1: the last entry again, unused); one wait per batch
        float4 p0[kBwdBatch], p1[kBwdBatch];
        float blue[kBwdBatch], slot[kBwdBatch];
        uint32_t gi[kBwdBatch], si[kBwdBatch];
        C.at<kBwdBatch>(jt, gi, si);
#pragma unroll
        for (int i = 0; i < kBwdBatch; ++i) {
            const float4 *rb = grec + kGRecF4 * (size_t)gi[i];
            p0[i] = rb[0];
            p1[i] = rb[1];
            blue[i] = rb[2].x;
            slot[i] = __uint_as_float(si[i]);
        }
#pragma unroll
        for (int i = 0; i < kBwdBatch; ++i)
            asm volatile("" ::"s"(p0[i].x), "s"(p0[i].y), "s"(p0[i].z), "s"(p0[i].w), "s"(p1[i].x), "s"(p1[i].y),
                         "s"(p1[i].z), "s"(p1[i].w), "s"(blue[i]), "s"(slot[i]));
        const uint32_t cnt = min((uint32_t)kBwdBatch, j1 - jt);
        float v[kBwdBatch * kFields];
        bool any = false;
#pragma unroll
        for (int i = 0; i < kBwdBatch; ++i) {
            float *o = v + kFields * i;
            const float dx = fx - p0[i].x, dy = fy - p0[i].y;
            const float raw = exp2_fast(exponent(p0[i], p1[i], dx, dy));
            // the forward pass's alpha and T, bit for bit
            const float alpha = fminf(alpha_max, raw);
            const bool take = (uint32_t)i < cnt && jt + (uint32_t)i < jend && alpha >= alpha_min;
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
        uint32_t *dst_stamp = qstamp + my_slot;
        const bool writer = (uint32_t)row < cnt && lane_writes;
        jt += cnt;
        if (__ballot(any) == 0) continue;   // no pixel takes these records: slots left unstamped
        float fz, t8;
        reduce_4x9(v, nl, fz, t8);
        if (writer) {
            if (stamp_lane)
                *dst_stamp = epoch;
            else
                *dst = nl == 1 ? t8 : fz;
        }
    }
    C.finish();
}

}  // namespace gsr
