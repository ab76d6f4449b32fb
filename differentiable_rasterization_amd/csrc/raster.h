// Shared definitions of the forward and backward rasterization kernels.
//
// Layout: one 64-lane wave per 16x16 tile.  Lane l owns the four pixels of column
// l % 16, rows 4*(l / 16) .. 4*(l / 16) + 3 of the tile.  The tile's list is staged
// through LDS 64 entries at a time (one gather per lane); every lane then walks the
// batch reading each entry as an LDS broadcast, so one LDS read serves four pixels.
#pragma once

#include "common.h"

namespace gsr {

constexpr int kBatch = 64;
constexpr int kPix = 4;
constexpr float kLog2e = 1.4426950408889634f;

// One list entry in the form the inner loop uses.  The alpha exponent is evaluated
// base 2: with (dx, dy) = pixel centre - mean,
//   o exp(-A dx^2/2 - B dx dy - C dy^2/2) = exp2(a dx^2 + b dx dy + c dy^2 + l)
// where a = -log2(e) A / 2, b = -log2(e) B, c = -log2(e) C / 2, l = log2(o).
struct Entry {
    float4 p0;   // u, v, a, b
    float4 p1;   // c, l, r, g
    float4 p2;   // blue, A, B, C
    float4 p3;   // 1/o, -, -, -
};

__device__ __forceinline__ Entry make_entry(uint32_t g, const float2 *__restrict__ means2d,
                                            const float4 *__restrict__ conic_o, const float *__restrict__ color)
{
    const float2 m = means2d[g];
    const float4 co = conic_o[g];
    const float r = color[3 * (size_t)g], gg = color[3 * (size_t)g + 1], b = color[3 * (size_t)g + 2];
    Entry e;
    e.p0 = make_float4(m.x, m.y, -0.5f * kLog2e * co.x, -kLog2e * co.y);
    e.p1 = make_float4(-0.5f * kLog2e * co.z, __builtin_amdgcn_logf(co.w), r, gg);
    e.p2 = make_float4(b, co.x, co.y, co.z);
    e.p3 = make_float4(__builtin_amdgcn_rcpf(co.w), 0.0f, 0.0f, 0.0f);
    return e;
}

// exp2 exponent of entry (p0, p1) at a pixel: `base` = a dx^2 + l and `bdx` = b dx are
// shared by the four pixels of a lane (same column).
__device__ __forceinline__ float exponent(float base, float bdx, float c, float dy)
{
    return fmaf(c * dy, dy, fmaf(bdx, dy, base));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gsr
