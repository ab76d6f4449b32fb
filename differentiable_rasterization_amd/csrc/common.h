// Internal helpers of libgsmi (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gs.h"

namespace gsi {

// Records `s` with a printf-style message in the thread-local error slot and returns it.
gs_status fail(gs_status s, const char *fmt, ...);

// Converts a HIP error into GS_ERR_HIP (with the runtime's text), or returns GS_OK.
gs_status hip_check(hipError_t e, const char *what);

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kWave = 64;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int tiles_x(int w) { return (w + GS_TILE - 1) / GS_TILE; }
inline int tiles_y(int h) { return (h + GS_TILE - 1) / GS_TILE; }

// Blocks are handed to the 8 XCDs of the chip round-robin (block b -> XCD b % 8).
// Mapping block b to tile (b % 8) * per_xcd + b / 8 gives every XCD one contiguous
// band of tiles, so neighbouring tiles, which share most of their Gaussians, hit the
// same L2.  Grid size: 8 * per_xcd; blocks past the last tile exit.
constexpr int kXcds = 8;
inline int xcd_per(int tiles) { return (tiles + kXcds - 1) / kXcds; }

// Plane strides of the parameter groups and of gradient / moment sets (0 in the struct: n).
inline int64_t param_ld(const gs_gaussians *g) { return g->ld ? g->ld : g->n; }
inline int64_t grads_ld(const gs_param_grads *pg, int64_t n) { return pg->ld ? pg->ld : n; }

gs_status check_camera(const gs_camera *cam);
gs_status check_params(const gs_raster_params *p);

}  // namespace gsi

#define GS_HIP(expr)                                                  \
    do {                                                              \
        gs_status s_ = gsi::hip_check((expr), #expr);                 \
        if (s_ != GS_OK) return s_;                                   \
    } while (0)

#define GS_LAUNCH_CHECK(name)                                         \
    do {                                                              \
        gs_status s_ = gsi::hip_check(hipGetLastError(), name);       \
        if (s_ != GS_OK) return s_;                                   \
    } while (0)

// ------------------------------------------------------------------ device helpers

namespace gsd {

__device__ __forceinline__ float f_from_i(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int i_from_f(float x) { return __builtin_bit_cast(int, x); }

// DPP controls (gfx9 encoding).
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// Sum over the 64 lanes of a wave; the total lands in lane 63.  Must be called with
// every lane of the wave active.  Four DPP steps sum each 16-lane row, two row
// broadcasts fold the rows into the last one.
__device__ __forceinline__ float wave_sum_to_lane63(float v)
{
    v += f_from_i(__builtin_amdgcn_mov_dpp(i_from_f(v), kQuadSwap1, 0xF, 0xF, false));
    v += f_from_i(__builtin_amdgcn_mov_dpp(i_from_f(v), kQuadSwap2, 0xF, 0xF, false));
    v += f_from_i(__builtin_amdgcn_mov_dpp(i_from_f(v), kRowHalfMirror, 0xF, 0xF, false));
    v += f_from_i(__builtin_amdgcn_mov_dpp(i_from_f(v), kRowMirror, 0xF, 0xF, false));
    v += f_from_i(__builtin_amdgcn_update_dpp(0, i_from_f(v), kRowBcast15, 0xA, 0xF, false));
    v += f_from_i(__builtin_amdgcn_update_dpp(0, i_from_f(v), kRowBcast31, 0xC, 0xF, false));
    return v;
}

// Integer sum over the 64 lanes of a wave; the total lands in lane 63.  Same pattern.
__device__ __forceinline__ unsigned wave_sum_u32_to_lane63(unsigned v)
{
    v += (unsigned)__builtin_amdgcn_mov_dpp((int)v, kQuadSwap1, 0xF, 0xF, false);
    v += (unsigned)__builtin_amdgcn_mov_dpp((int)v, kQuadSwap2, 0xF, 0xF, false);
    v += (unsigned)__builtin_amdgcn_mov_dpp((int)v, kRowHalfMirror, 0xF, 0xF, false);
    v += (unsigned)__builtin_amdgcn_mov_dpp((int)v, kRowMirror, 0xF, 0xF, false);
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kRowBcast15, 0xA, 0xF, false);
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kRowBcast31, 0xC, 0xF, false);
    return v;
}

// Maximum over the 64 lanes of a wave, returned to every lane (uniform).
__device__ __forceinline__ int wave_max_i32(int v)
{
    v = max(v, __builtin_amdgcn_mov_dpp(v, kQuadSwap1, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_mov_dpp(v, kQuadSwap2, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_mov_dpp(v, kRowHalfMirror, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_mov_dpp(v, kRowMirror, 0xF, 0xF, false));
    int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ unsigned lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ unsigned rank_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

// One bias-corrected Adam step of one scalar (step = lr / (1 - b1^t), inv_bc2 =
// 1 / (1 - b2^t)); every Adam path of the library uses this, so they agree bit for bit.
__device__ __forceinline__ void adam_update(float &p, float g, float &m, float &v, float b1, float b2, float inv_bc2,
                                            float eps, float step)
{
    m = fmaf(b1, m, (1.0f - b1) * g);
    v = fmaf(b2, v, (1.0f - b2) * g * g);
    p -= step * m / (__fsqrt_rn(v * inv_bc2) + eps);
}

// Tile rectangle [x0,x1) x [y0,y1) touched by the box [u-rx, u+rx] x [v-ry, v+ry],
// float32 arithmetic (division by 16 is exact), clamped to the tile grid.
__device__ __forceinline__ void tile_rect(float u, float v, int rx, int ry, int tx, int ty,
                                          int &x0, int &x1, int &y0, int &y1)
{
    float a = floorf(__fsub_rn(u, (float)rx) * 0.0625f);
    float b = floorf(__fadd_rn(u, (float)rx) * 0.0625f) + 1.0f;
    float c = floorf(__fsub_rn(v, (float)ry) * 0.0625f);
    float d = floorf(__fadd_rn(v, (float)ry) * 0.0625f) + 1.0f;
    x0 = (int)fminf(fmaxf(a, 0.0f), (float)tx);
    x1 = (int)fminf(fmaxf(b, 0.0f), (float)tx);
    y0 = (int)fminf(fmaxf(c, 0.0f), (float)ty);
    y1 = (int)fminf(fmaxf(d, 0.0f), (float)ty);
}

}  // namespace gsd
