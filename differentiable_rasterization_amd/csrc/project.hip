// Projection of 3D Gaussians to 2D records with SH colour (forward), and its
// backward through projection and colour evaluation.
//
// Forward, per Gaussian (one thread each, coalesced structure-of-arrays loads):
//   s = exp(log_s), o = sigmoid(logit), q^ = q / |q|, R = R(q^)
//   Sigma = M M^T, M = R diag(s)                       (Splaxel, section 2)
//   p = W mu + t;  u = fx X/Z + cx, v = fy Y/Z + cy     (frustum culling by the mean)
//   Sigma2D = T Sigma T^T, T = J W, J the pinhole Jacobian at p   (Splaxel, section 2)
//   conic = Sigma2D^-1; radii from the alpha >= alpha_min ellipse
//   colour = sum_k sh_k Y_k(v^), v^ the unit vector from the camera centre to mu
//     ("Scaling 3D Gaussian Splatting with Distributed Compute", walkthrough step 4)
// The geometric chain runs in double (it is memory bound, so this costs no time on
// MI355X) and is rounded once to the float32 record.  SH evaluation runs in float.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "raster.h"

// No implicit multiply-add contraction in this file: the forward projection, its recomputation
// in the backward kernels and the fused step must round identically (the same cull
// decisions and records in every kernel), which per-kernel contraction choices would not
// guarantee.  Explicit fmaf calls stay fused.
#pragma clang fp contract(off)

namespace {

struct CamD {
    double R[9];
    double t[3];
    double fx, fy, cx, cy;
    double campos[3];
    double near_z;
    float r20, r21, r22, t2;
    int W, H;
};

CamD make_cam(const gs_camera *c)
{
    CamD d;
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j) d.R[3 * i + j] = c->viewmat[4 * i + j];
        d.t[i] = c->viewmat[4 * i + 3];
    }
    d.fx = c->fx; d.fy = c->fy; d.cx = c->cx; d.cy = c->cy;
    for (int j = 0; j < 3; ++j)
        d.campos[j] = -(d.R[0 * 3 + j] * d.t[0] + d.R[1 * 3 + j] * d.t[1] + d.R[2 * 3 + j] * d.t[2]);
    d.near_z = c->near_z;
    d.r20 = c->viewmat[8]; d.r21 = c->viewmat[9]; d.r22 = c->viewmat[10]; d.t2 = c->viewmat[11];
    d.W = c->width; d.H = c->height;
    return d;
}

// Real orthonormal SH basis up to degree 3 as Cartesian polynomials on the unit
// sphere (no Condon-Shortley phase), index k = l*l + l + m.  Normalisations:
//   l=0: 1/(2 sqrt(pi));  l=1: sqrt(3/(4 pi))
//   l=2: sqrt(15/pi)/2 (xy, yz, xz), sqrt(5/pi)/4 (3z^2-1), sqrt(15/pi)/4 (x^2-y^2)
//   l=3: sqrt(35/(2 pi))/4 (y(3x^2-y^2), x(x^2-3y^2)), sqrt(105/pi)/2 (xyz),
//        sqrt(21/(2 pi))/4 (y(5z^2-1), x(5z^2-1)), sqrt(7/pi)/4 (z(5z^2-3)),
//        sqrt(105/pi)/4 (z(x^2-y^2))
constexpr float kSH0 = 0.28209479177387814f;
constexpr float kSH1 = 0.48860251190291992f;
constexpr float kSH2a = 1.0925484305920792f;
constexpr float kSH2b = 0.31539156525252005f;
constexpr float kSH2c = 0.54627421529603959f;
constexpr float kSH3a = 0.59004358992664352f;
constexpr float kSH3b = 2.8906114426405538f;
constexpr float kSH3c = 0.45704579946446572f;
constexpr float kSH3d = 0.37317633259011540f;
constexpr float kSH3e = 1.4453057213202769f;

template <int DEG>
__device__ __forceinline__ void sh_basis(float x, float y, float z, float *Y)
{
    Y[0] = kSH0;
    if (DEG >= 1) { Y[1] = kSH1 * y; Y[2] = kSH1 * z; Y[3] = kSH1 * x; }
    if (DEG >= 2) {
        const float xx = x * x, yy = y * y, zz = z * z;
        Y[4] = kSH2a * x * y; Y[5] = kSH2a * y * z; Y[6] = kSH2b * (3.0f * zz - 1.0f);
        Y[7] = kSH2a * x * z; Y[8] = kSH2c * (xx - yy);
        if (DEG >= 3) {
            Y[9] = kSH3a * y * (3.0f * xx - yy);
            Y[10] = kSH3b * x * y * z;
            Y[11] = kSH3c * y * (5.0f * zz - 1.0f);
            Y[12] = kSH3d * z * (5.0f * zz - 3.0f);
            Y[13] = kSH3c * x * (5.0f * zz - 1.0f);
            Y[14] = kSH3e * z * (xx - yy);
            Y[15] = kSH3a * x * (xx - 3.0f * yy);
        }
    }
}

// Gradient of sum_k w_k Y_k(x, y, z) with respect to (x, y, z) (polynomial extension;
// its tangential part is the derivative on the sphere).
template <int DEG>
__device__ __forceinline__ void sh_grad(float x, float y, float z, const float *w, float &gx, float &gy, float &gz)
{
    gx = gy = gz = 0.0f;
    if (DEG >= 1) { gy += kSH1 * w[1]; gz += kSH1 * w[2]; gx += kSH1 * w[3]; }
    if (DEG >= 2) {
        gx += kSH2a * (y * w[4] + z * w[7]) + 2.0f * kSH2c * x * w[8];
        gy += kSH2a * (x * w[4] + z * w[5]) - 2.0f * kSH2c * y * w[8];
        gz += kSH2a * (y * w[5] + x * w[7]) + 6.0f * kSH2b * z * w[6];
        if (DEG >= 3) {
            const float xx = x * x, yy = y * y, zz = z * z;
            gx += kSH3a * 6.0f * x * y * w[9] + kSH3b * y * z * w[10] + kSH3c * (5.0f * zz - 1.0f) * w[13]
                + kSH3e * 2.0f * x * z * w[14] + kSH3a * 3.0f * (xx - yy) * w[15];
            gy += kSH3a * 3.0f * (xx - yy) * w[9] + kSH3b * x * z * w[10] + kSH3c * (5.0f * zz - 1.0f) * w[11]
                - kSH3e * 2.0f * y * z * w[14] - kSH3a * 6.0f * x * y * w[15];
            gz += kSH3b * x * y * w[10] + kSH3c * 10.0f * y * z * w[11] + kSH3d * (15.0f * zz - 3.0f) * w[12]
                + kSH3c * 10.0f * x * z * w[13] + kSH3e * (xx - yy) * w[14];
        }
    }
}

// Everything the forward computes for one Gaussian, kept for the backward.
// What the projection backward needs of the forward; the matrices R(q^), M, Sigma and T are
// recomputed from these by the same code (rot_q, cov3d, jw), so they need not stay live.
struct Proj {
    bool vis;
    float key;
    double s[3], q[4], qnorm, o;
    double X, Y, Z, u, v;
    double a, b, c, A, B, C;
    double dist;
    float dir[3];        // unit view direction
    int rx, ry;
};

// R(q^) of the unit quaternion (w, x, y, z), row-major.
__device__ __forceinline__ void rot_q(double w, double x, double y, double z, double (&R)[9])
{
    R[0] = 1.0 - 2.0 * (y * y + z * z); R[1] = 2.0 * (x * y - w * z);       R[2] = 2.0 * (x * z + w * y);
    R[3] = 2.0 * (x * y + w * z);       R[4] = 1.0 - 2.0 * (x * x + z * z); R[5] = 2.0 * (y * z - w * x);
    R[6] = 2.0 * (x * z - w * y);       R[7] = 2.0 * (y * z + w * x);       R[8] = 1.0 - 2.0 * (x * x + y * y);
}

// M = R diag(s) and Sigma = M M^T (xx, xy, xz, yy, yz, zz).
__device__ __forceinline__ void cov3d(const double (&R)[9], const double (&s)[3], double (&M)[9], double (&Sig)[6])
{
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) M[3 * r + c] = R[3 * r + c] * s[c];
    Sig[0] = M[0] * M[0] + M[1] * M[1] + M[2] * M[2];
    Sig[1] = M[0] * M[3] + M[1] * M[4] + M[2] * M[5];
    Sig[2] = M[0] * M[6] + M[1] * M[7] + M[2] * M[8];
    Sig[3] = M[3] * M[3] + M[4] * M[4] + M[5] * M[5];
    Sig[4] = M[3] * M[6] + M[4] * M[7] + M[5] * M[8];
    Sig[5] = M[6] * M[6] + M[7] * M[7] + M[8] * M[8];
}

__device__ __forceinline__ bool finite_d(double x) { return __builtin_isfinite(x); }

// The camera-independent transcendental values of one Gaussian: |q|, the scales, the
// opacity and 2 ln(o / alpha_min).  ok is false for a Gaussian no camera keeps (non-finite
// input, |q| = 0, opacity below alpha_min).
struct ProjScalars {
    bool ok;
    double qnorm, s[3], o, lnr;
};

__device__ __forceinline__ void project_scalars(double mx, double my, double mz, double l0, double l1, double l2,
                                                double q0, double q1, double q2, double q3, double logit,
                                                bool sh_finite, double alpha_min, ProjScalars &S)
{
    S.ok = false;
    if (!(finite_d(mx) && finite_d(my) && finite_d(mz) && finite_d(l0) && finite_d(l1) && finite_d(l2) &&
          finite_d(q0) && finite_d(q1) && finite_d(q2) && finite_d(q3) && finite_d(logit) && sh_finite))
        return;
    S.qnorm = sqrt(q0 * q0 + q1 * q1 + q2 * q2 + q3 * q3);
    if (!(S.qnorm > 0.0)) return;
    S.s[0] = exp(l0); S.s[1] = exp(l1); S.s[2] = exp(l2);
    S.o = 1.0 / (1.0 + exp(-logit));
    const double o32 = (double)(float)S.o;
    if (!(o32 >= alpha_min)) return;
    S.lnr = 2.0 * log(o32 / alpha_min);
    S.ok = true;
}

// T = J W (2 x 3): the projection's Jacobian at camera-space (X, Y, Z) times the rotation.
__device__ __forceinline__ void jw(const CamD &cam, double X, double Y, double Z, double (&T)[6])
{
    const double iz = 1.0 / Z;
    const double j00 = cam.fx * iz, j02 = -cam.fx * X * iz * iz;
    const double j11 = cam.fy * iz, j12 = -cam.fy * Y * iz * iz;
    for (int c = 0; c < 3; ++c) {
        T[c] = j00 * cam.R[c] + j02 * cam.R[6 + c];
        T[3 + c] = j11 * cam.R[3 + c] + j12 * cam.R[6 + c];
    }
}

// The projection for one camera, from the Gaussian's parameters and its ProjScalars.
__device__ __forceinline__ void project_view(const CamD &cam, double mx, double my, double mz, float fmx, float fmy,
                                             float fmz, double q0, double q1, double q2, double q3,
                                             const ProjScalars &S, float depth_lo, float depth_hi, Proj &P)
{
    P.vis = false;
    P.rx = P.ry = 0;
    // camera-space depth as the float32 key: each step rounded explicitly
    P.key = __fadd_rn(__fmaf_rn(cam.r22, fmz, __fmaf_rn(cam.r21, fmy, __fmul_rn(cam.r20, fmx))), cam.t2);
    if (!S.ok) return;
    if (!(P.key >= depth_lo && P.key < depth_hi)) return;
    P.qnorm = S.qnorm;
    P.X = cam.R[0] * mx + cam.R[1] * my + cam.R[2] * mz + cam.t[0];
    P.Y = cam.R[3] * mx + cam.R[4] * my + cam.R[5] * mz + cam.t[1];
    P.Z = cam.R[6] * mx + cam.R[7] * my + cam.R[8] * mz + cam.t[2];
    if (!(P.Z > cam.near_z)) return;
    P.u = cam.fx * P.X / P.Z + cam.cx;
    P.v = cam.fy * P.Y / P.Z + cam.cy;
    if (!(P.u >= 0.0 && P.u < (double)cam.W && P.v >= 0.0 && P.v < (double)cam.H)) return;

    const double iq = 1.0 / P.qnorm;
    const double w = q0 * iq, x = q1 * iq, y = q2 * iq, z = q3 * iq;
    P.q[0] = w; P.q[1] = x; P.q[2] = y; P.q[3] = z;
    P.s[0] = S.s[0]; P.s[1] = S.s[1]; P.s[2] = S.s[2];
    double R[9], M[9], Sg[6], T[6];
    rot_q(w, x, y, z, R);
    cov3d(R, P.s, M, Sg);
    jw(cam, P.X, P.Y, P.Z, T);
    // (T Sigma) rows
    double ts0[3], ts1[3];
    ts0[0] = T[0] * Sg[0] + T[1] * Sg[1] + T[2] * Sg[2];
    ts0[1] = T[0] * Sg[1] + T[1] * Sg[3] + T[2] * Sg[4];
    ts0[2] = T[0] * Sg[2] + T[1] * Sg[4] + T[2] * Sg[5];
    ts1[0] = T[3] * Sg[0] + T[4] * Sg[1] + T[5] * Sg[2];
    ts1[1] = T[3] * Sg[1] + T[4] * Sg[3] + T[5] * Sg[4];
    ts1[2] = T[3] * Sg[2] + T[4] * Sg[4] + T[5] * Sg[5];
    P.a = ts0[0] * T[0] + ts0[1] * T[1] + ts0[2] * T[2];
    P.b = ts0[0] * T[3] + ts0[1] * T[4] + ts0[2] * T[5];
    P.c = ts1[0] * T[3] + ts1[1] * T[4] + ts1[2] * T[5];
    const double det = P.a * P.c - P.b * P.b;
    if (!(det > 0.0)) return;
    const double idet = 1.0 / det;
    P.A = P.c * idet; P.B = -P.b * idet; P.C = P.a * idet;

    P.o = S.o;
    const double lnr = S.lnr;
    double ex = ceil(sqrt(lnr * P.a)), ey = ceil(sqrt(lnr * P.c));
    ex = fmin(fmax(ex, 1.0), (double)GS_RADIUS_CAP);
    ey = fmin(fmax(ey, 1.0), (double)GS_RADIUS_CAP);
    P.rx = (int)ex; P.ry = (int)ey;

    const double dx = mx - cam.campos[0], dy = my - cam.campos[1], dz = mz - cam.campos[2];
    P.dist = sqrt(dx * dx + dy * dy + dz * dz);
    const double id = 1.0 / P.dist;
    P.dir[0] = (float)(dx * id); P.dir[1] = (float)(dy * id); P.dir[2] = (float)(dz * id);
    P.vis = true;
}

__device__ __forceinline__ void project_core(const CamD &cam, double mx, double my, double mz, float fmx,
                                             float fmy, float fmz, double l0, double l1, double l2, double q0,
                                             double q1, double q2, double q3, double logit, bool sh_finite,
                                             double alpha_min, float depth_lo, float depth_hi, Proj &P)
{
    ProjScalars S;
    project_scalars(mx, my, mz, l0, l1, l2, q0, q1, q2, q3, logit, sh_finite, alpha_min, S);
    project_view(cam, mx, my, mz, fmx, fmy, fmz, q0, q1, q2, q3, S, depth_lo, depth_hi, P);
}

// The conic and opacity of the raster record, as float: a = -A log2(e)/2, b = -B log2(e),
// c = -C log2(e)/2, l = log2 of the float32 opacity.
struct RecConic {
    float a, b, c, l;
};

__device__ __forceinline__ RecConic rec_conic(const Proj &P)
{
    constexpr double kL2e = 1.4426950408889634;
    const double o32 = (double)(float)P.o;
    return {(float)(-0.5 * kL2e * P.A), (float)(-kL2e * P.B), (float)(-0.5 * kL2e * P.C), (float)log2(o32)};
}

template <int K>
struct Params1 {   // one Gaussian's parameters as loaded
    float means[3], ls[3], q[4], logit, sh[3 * K];
};

// NT: non-temporal loads.  Measured faster in the end-of-step passes (whose parameter
// stores are non-temporal too) and slower in the standalone projection and projection
// backward, which keep ordinary loads.
// NT_SH: the SH coefficients too (false: ordinary loads, so that a second read soon after
// finds them in L2).
template <bool NT, int K, bool NT_SH = NT>
__device__ __forceinline__ void load_params(const float *__restrict__ means, const float *__restrict__ log_scales,
                                            const float *__restrict__ quats, const float *__restrict__ logits,
                                            const float *__restrict__ sh, int64_t n, int64_t i, Params1<K> &prm)
{
    // n: the plane stride of the parameter groups
    const auto ld = [](const float *p) { return NT ? __builtin_nontemporal_load(p) : *p; };
    const auto ld_sh = [](const float *p) { return NT_SH ? __builtin_nontemporal_load(p) : *p; };
    prm.means[0] = ld(means + i); prm.means[1] = ld(means + n + i); prm.means[2] = ld(means + 2 * n + i);
    prm.ls[0] = ld(log_scales + i); prm.ls[1] = ld(log_scales + n + i); prm.ls[2] = ld(log_scales + 2 * n + i);
    prm.q[0] = ld(quats + i); prm.q[1] = ld(quats + n + i); prm.q[2] = ld(quats + 2 * n + i);
    prm.q[3] = ld(quats + 3 * n + i);
    prm.logit = ld(logits + i);
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) prm.sh[k] = ld_sh(sh + (int64_t)k * n + i);
}

// The 11 scalars other than the SH coefficients (n: the plane stride), and the coefficients
// on their own, for kernels that load the latter only for visible Gaussians.
template <int K>
__device__ __forceinline__ void load_geometry(const float *__restrict__ means, const float *__restrict__ log_scales,
                                              const float *__restrict__ quats, const float *__restrict__ logits,
                                              int64_t n, int64_t i, Params1<K> &prm)
{
    prm.means[0] = means[i]; prm.means[1] = means[n + i]; prm.means[2] = means[2 * n + i];
    prm.ls[0] = log_scales[i]; prm.ls[1] = log_scales[n + i]; prm.ls[2] = log_scales[2 * n + i];
    prm.q[0] = quats[i]; prm.q[1] = quats[n + i]; prm.q[2] = quats[2 * n + i]; prm.q[3] = quats[3 * n + i];
    prm.logit = logits[i];
}

template <int K>
__device__ __forceinline__ void load_sh(const float *__restrict__ sh, int64_t n, int64_t i, Params1<K> &prm)
{
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) prm.sh[k] = sh[(int64_t)k * n + i];
}

template <int K>
__device__ __forceinline__ bool sh_finite(const Params1<K> &prm)
{
    bool f = true;
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) f = f && __builtin_isfinite(prm.sh[k]);
    return f;
}

// The projection's outputs (gs_projected): the depth key, the radii and the raster record of
// every Gaussian, and optionally the plain record fields as planes of n floats.
struct ProjOut {
    float *means2d, *conic_o, *color;   // [2][n], [4][n], [3][n]; NULL: that group is not written
    float *depth;
    int2 *radii;
    float4 *rec;
    int64_t n;
};

// Projects Gaussian i with parameters prm and stores its projected record: the one
// definition both gs_project and the projection fused into the end of a step use.
template <int K>
__device__ __forceinline__ void params_scalars(const Params1<K> &prm, float alpha_min, ProjScalars &S)
{
    project_scalars(prm.means[0], prm.means[1], prm.means[2], prm.ls[0], prm.ls[1], prm.ls[2], prm.q[0], prm.q[1],
                    prm.q[2], prm.q[3], prm.logit, sh_finite(prm), (double)alpha_min, S);
}

template <int DEG>
__device__ __forceinline__ void project_store_s(const Params1<(DEG + 1) * (DEG + 1)> &prm, const ProjScalars &S,
                                                const CamD &cam, float depth_lo, float depth_hi, int64_t i,
                                                const ProjOut &po);

template <int DEG>
__device__ __forceinline__ void project_store(const Params1<(DEG + 1) * (DEG + 1)> &prm, const CamD &cam,
                                              float alpha_min, float depth_lo, float depth_hi, int64_t i,
                                              const ProjOut &po)
{
    ProjScalars S;
    params_scalars(prm, alpha_min, S);
    project_store_s<DEG>(prm, S, cam, depth_lo, depth_hi, i, po);
}

// The float fields of a visible Gaussian's outputs, as rounded from its projection.
struct RecFields {
    float u, v, A, B, C, o;
    RecConic rc;   // raster-ready: conic scaled for exp2, log2 of the stored opacity
    int rx, ry;
};

__device__ __forceinline__ RecFields rec_fields(const Proj &P)
{
    return {(float)P.u, (float)P.v, (float)P.A, (float)P.B, (float)P.C, (float)P.o, rec_conic(P), P.rx, P.ry};
}

// The record of a visible Gaussian with colour (r, g, b); its plain fields (where requested)
// are stored on the way.
__device__ __forceinline__ void record_visible(const RecFields &F, float r, float g, float b, int64_t i,
                                               const ProjOut &po, float4 (&rec)[3])
{
    const int64_t n = po.n;
    if (po.means2d) {
        po.means2d[i] = F.u;
        po.means2d[n + i] = F.v;
    }
    if (po.conic_o) {
        po.conic_o[i] = F.A;
        po.conic_o[n + i] = F.B;
        po.conic_o[2 * n + i] = F.C;
        po.conic_o[3 * n + i] = F.o;
    }
    if (po.color) {
        po.color[i] = r;
        po.color[n + i] = g;
        po.color[2 * n + i] = b;
    }
    rec[0] = make_float4(F.u, F.v, F.rc.a, F.rc.b);
    rec[1] = make_float4(F.rc.c, F.rc.l, r, g);
    rec[2] = make_float4(b, __uint_as_float((uint32_t)i), __int_as_float(F.rx), __int_as_float(F.ry));
}

// The projected record of Gaussian i as three float4 of the raster record; depth, radii and
// the plain fields (where requested) are stored on the way.  A culled Gaussian's record is
// zero apart from its index (its radii are (0, 0)).
template <int DEG>
__device__ __forceinline__ void record_from(const Params1<(DEG + 1) * (DEG + 1)> &prm, const Proj &P, int64_t i,
                                            const ProjOut &po, float4 (&rec)[3])
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    po.depth[i] = P.key;
    po.radii[i] = make_int2(P.rx, P.ry);
    rec[0] = rec[1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    rec[2] = make_float4(0.0f, __uint_as_float((uint32_t)i), 0.0f, 0.0f);
    if (!P.vis) return;
    float Y[K];
    sh_basis<DEG>(P.dir[0], P.dir[1], P.dir[2], Y);
    float r = 0.0f, g = 0.0f, b = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        r = fmaf(prm.sh[3 * k + 0], Y[k], r);
        g = fmaf(prm.sh[3 * k + 1], Y[k], g);
        b = fmaf(prm.sh[3 * k + 2], Y[k], b);
    }
    record_visible(rec_fields(P), r, g, b, i, po, rec);
}

template <int DEG>
__device__ __forceinline__ void project_record(const Params1<(DEG + 1) * (DEG + 1)> &prm, const ProjScalars &S,
                                               const CamD &cam, float depth_lo, float depth_hi, int64_t i,
                                               const ProjOut &po, float4 (&rec)[3])
{
    Proj P;
    const float fmx = prm.means[0], fmy = prm.means[1], fmz = prm.means[2];
    project_view(cam, fmx, fmy, fmz, fmx, fmy, fmz, prm.q[0], prm.q[1], prm.q[2], prm.q[3], S, depth_lo, depth_hi, P);
    record_from<DEG>(prm, P, i, po, rec);
}

// project_store with the Gaussian's camera-independent values already computed.  The record
// goes straight from registers (three 16-byte stores 48 bytes apart per lane; staging a
// block's records through LDS for contiguous stores measured no faster).
template <int DEG>
__device__ __forceinline__ void project_store_s(const Params1<(DEG + 1) * (DEG + 1)> &prm, const ProjScalars &S,
                                                const CamD &cam, float depth_lo, float depth_hi, int64_t i,
                                                const ProjOut &po)
{
    float4 rec[3];
    project_record<DEG>(prm, S, cam, depth_lo, depth_hi, i, po, rec);
    po.rec[3 * i + 0] = rec[0];
    po.rec[3 * i + 1] = rec[1];
    po.rec[3 * i + 2] = rec[2];
}

template <int DEG>
__global__ __launch_bounds__(256) void k_project(const float *__restrict__ means, const float *__restrict__ log_scales,
                                                 const float *__restrict__ quats, const float *__restrict__ logits,
                                                 const float *__restrict__ sh, int64_t n, int64_t ldp, CamD cam,
                                                 float alpha_min, float depth_lo, float depth_hi, ProjOut po)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    // The geometry decides visibility first (with the SH taken as finite); only the visible
    // lanes load their SH coefficients, and non-finite ones cull the Gaussian then, which
    // gives what project_store gives (a culled Gaussian's depth key does not depend on them).
    Params1<K> prm;
    load_geometry(means, log_scales, quats, logits, ldp, i, prm);
    ProjScalars S;
    project_scalars(prm.means[0], prm.means[1], prm.means[2], prm.ls[0], prm.ls[1], prm.ls[2], prm.q[0], prm.q[1],
                    prm.q[2], prm.q[3], prm.logit, true, (double)alpha_min, S);
    Proj P;
    const float fmx = prm.means[0], fmy = prm.means[1], fmz = prm.means[2];
    project_view(cam, fmx, fmy, fmz, fmx, fmy, fmz, prm.q[0], prm.q[1], prm.q[2], prm.q[3], S, depth_lo, depth_hi, P);
    if (P.vis) {
        load_sh(sh, ldp, i, prm);
        if (!sh_finite(prm)) {
            P.vis = false;
            P.rx = P.ry = 0;
        }
    }
    float4 rec[3];
    record_from<DEG>(prm, P, i, po, rec);
    po.rec[3 * i + 0] = rec[0];
    po.rec[3 * i + 1] = rec[1];
    po.rec[3 * i + 2] = rec[2];
}

// Backward through projection and colour evaluation (ByteSplat, section 2.1: the
// aggregated screen-space gradients are propagated through projection and colour
// evaluation to the 3D parameters).  Exact chain rule of project_core; the float
// rounding of the record is treated as the identity.  The gradients of one Gaussian are
// collected in registers (the SH gradients as Y_k(v^) and dL/dc, their product formed
// where it is used) and handed with the current parameter values to a sink: GradSink
// stores them, AdamSink applies the Adam update at once.
template <int K>
struct Grad3 {
    float means[3], ls[3], q[4], logit;
    float Y[K], gc[3];
    __device__ float sh(int plane) const { return Y[plane / 3] * gc[plane % 3]; }
};

struct GradSink {
    float *d_means, *d_ls, *d_q, *d_logit, *d_sh;
    int64_t n;   // the plane stride of the gradient planes
    template <int K>
    __device__ void flush(int64_t i, const Grad3<K> &g, const Params1<K> &) const
    {
        for (int j = 0; j < 3; ++j) d_means[j * n + i] = g.means[j];
        for (int j = 0; j < 3; ++j) d_ls[j * n + i] = g.ls[j];
        for (int j = 0; j < 4; ++j) d_q[j * n + i] = g.q[j];
        d_logit[i] = g.logit;
#pragma unroll
        for (int k = 0; k < 3 * K; ++k) d_sh[(int64_t)k * n + i] = g.sh(k);
    }
};

// Planes per chunk of the SH update: the largest divisor of the plane count up to 12 (3,
// 12, 9 and 12 planes for degrees 0-3), so that the chunks tile the planes exactly.
constexpr int sh_chunk(int planes)
{
    for (int c = 12; c > 1; --c)
        if (planes % c == 0) return c;
    return 1;
}

// The same for the single-view update, which also holds each chunk's parameter values:
// chunks of at most 4 planes.
constexpr int view_chunk(int planes)
{
    for (int c = 4; c > 1; --c)
        if (planes % c == 0) return c;
    return 1;
}

// Adam over the parameter scalars of one Gaussian, a chunk of planes at a time: every
// moment load of a chunk is issued before any store, so the loads overlap, and the moments
// of the next chunk are loaded before the current chunk is updated and stored, so that a
// chunk's loads are in flight during the previous chunk's arithmetic and stores.
struct AdamSink {
    float *p[5], *m[5], *v[5];   // means, log_scales, quats, opacity_logits, sh
    int64_t n;                   // the plane stride of p, m and v
    float st[6];                 // lr / (1 - b1^t): means, log_scales, quats, opacity, sh DC, sh rest
    float b1, b2, inv_bc2, eps;

    template <int N>
    __device__ void load_mv(const int (&grp)[N], const int (&plane)[N], int64_t i, float (&mv)[N],
                            float (&vv)[N]) const
    {
#pragma unroll
        for (int c = 0; c < N; ++c) {
            const int64_t idx = (int64_t)plane[c] * n + i;
            mv[c] = __builtin_nontemporal_load(m[grp[c]] + idx);
            vv[c] = __builtin_nontemporal_load(v[grp[c]] + idx);
        }
    }

    // pv: the parameter values in, the updated values out
    template <int N>
    __device__ void update(const int (&grp)[N], const int (&plane)[N], const float (&g)[N], float (&pv)[N],
                           const float (&step)[N], float (&mv)[N], float (&vv)[N], int64_t i) const
    {
#pragma unroll
        for (int c = 0; c < N; ++c) {
            gsd::adam_update(pv[c], g[c], mv[c], vv[c], b1, b2, inv_bc2, eps, step[c]);
            const int64_t idx = (int64_t)plane[c] * n + i;
            __builtin_nontemporal_store(pv[c], p[grp[c]] + idx);
            __builtin_nontemporal_store(mv[c], m[grp[c]] + idx);
            __builtin_nontemporal_store(vv[c], v[grp[c]] + idx);
        }
    }

    // Updates and stores every parameter scalar of Gaussian i; P holds the updated values
    // afterwards.  Grad: Grad3 or GradSum (means, ls, q, logit and sh(plane)).
    template <class Grad, int K>
    __device__ void flush(int64_t i, const Grad &g, Params1<K> &P) const
    {
        constexpr int kChunk = sh_chunk(3 * K);
        static_assert((3 * K) % kChunk == 0, "the chunks must tile the SH planes exactly");
        // means, log_scales, quats, opacity: 11 scalars
        const int grp[11] = {0, 0, 0, 1, 1, 1, 2, 2, 2, 2, 3};
        const int pl[11] = {0, 1, 2, 0, 1, 2, 0, 1, 2, 3, 0};
        float m11[11], v11[11];
        load_mv(grp, pl, i, m11, v11);
        int sgrp[kChunk], spl[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            sgrp[c] = 4;
            spl[c] = c;
        }
        float msh[kChunk], vsh[kChunk];
        load_mv(sgrp, spl, i, msh, vsh);   // the first SH chunk
        {
            const float gg[11] = {g.means[0], g.means[1], g.means[2], g.ls[0], g.ls[1], g.ls[2],
                                  g.q[0], g.q[1], g.q[2], g.q[3], g.logit};
            float pv[11] = {P.means[0], P.means[1], P.means[2], P.ls[0], P.ls[1], P.ls[2],
                            P.q[0], P.q[1], P.q[2], P.q[3], P.logit};
            const float sp[11] = {st[0], st[0], st[0], st[1], st[1], st[1], st[2], st[2], st[2], st[2], st[3]};
            update(grp, pl, gg, pv, sp, m11, v11, i);
            P.means[0] = pv[0]; P.means[1] = pv[1]; P.means[2] = pv[2];
            P.ls[0] = pv[3]; P.ls[1] = pv[4]; P.ls[2] = pv[5];
            P.q[0] = pv[6]; P.q[1] = pv[7]; P.q[2] = pv[8]; P.q[3] = pv[9];
            P.logit = pv[10];
        }
#pragma unroll
        for (int c0 = 0; c0 < 3 * K; c0 += kChunk) {
            float mnx[kChunk], vnx[kChunk];
            if (c0 + kChunk < 3 * K) {   // the next chunk's moments
                int npl[kChunk];
#pragma unroll
                for (int c = 0; c < kChunk; ++c) npl[c] = c0 + kChunk + c;
                load_mv(sgrp, npl, i, mnx, vnx);
            }
            int cpl[kChunk];
            float gg[kChunk], pv[kChunk], sp[kChunk];
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                cpl[c] = c0 + c;
                gg[c] = g.sh(c0 + c);
                pv[c] = P.sh[c0 + c];
                sp[c] = c0 + c < 3 ? st[4] : st[5];
            }
            update(sgrp, cpl, gg, pv, sp, msh, vsh, i);
#pragma unroll
            for (int c = 0; c < kChunk; ++c) P.sh[c0 + c] = pv[c];
            if (c0 + kChunk < 3 * K) {
#pragma unroll
                for (int c = 0; c < kChunk; ++c) {
                    msh[c] = mnx[c];
                    vsh[c] = vnx[c];
                }
            }
        }
    }

    // The update of the single-view end of step, shaped to keep few values live: the SH
    // coefficients are read back from the wave's LDS copy a chunk at a time,
    // the SH gradients Y_k(dir) dc are formed from the view direction (vis false: zero), and
    // with NEXT the updated Gaussian is projected for next_cam on the way: its geometry right
    // after the 11 other scalars, its colour summed over the updated SH chunks in the order
    // project_record takes, and a non-finite updated coefficient culls it as there.  Every
    // value equals what flush followed by project_store gives.
    template <int DEG, bool NEXT>
    __device__ void flush_view(int64_t i, const Grad3<(DEG + 1) * (DEG + 1)> &g, bool vis, const float (&dir)[3],
                               Params1<(DEG + 1) * (DEG + 1)> &P, float (*shs)[64], float alpha_min, float depth_lo,
                               float depth_hi, const CamD &next_cam, const ProjOut &next) const
    {
        constexpr int K = (DEG + 1) * (DEG + 1);
        constexpr int kC = view_chunk(3 * K);
        const int grp[11] = {0, 0, 0, 1, 1, 1, 2, 2, 2, 2, 3};
        const int pl[11] = {0, 1, 2, 0, 1, 2, 0, 1, 2, 3, 0};
        float m11[11], v11[11];
        load_mv(grp, pl, i, m11, v11);
        int sgrp[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) sgrp[c] = 4;
        float msh[kC], vsh[kC], psh[kC];
        {
            const float gg[11] = {g.means[0], g.means[1], g.means[2], g.ls[0], g.ls[1], g.ls[2],
                                  g.q[0], g.q[1], g.q[2], g.q[3], g.logit};
            float pv[11] = {P.means[0], P.means[1], P.means[2], P.ls[0], P.ls[1], P.ls[2],
                            P.q[0], P.q[1], P.q[2], P.q[3], P.logit};
            const float sp[11] = {st[0], st[0], st[0], st[1], st[1], st[1], st[2], st[2], st[2], st[2], st[3]};
            update(grp, pl, gg, pv, sp, m11, v11, i);
            P.means[0] = pv[0]; P.means[1] = pv[1]; P.means[2] = pv[2];
            P.ls[0] = pv[3]; P.ls[1] = pv[4]; P.ls[2] = pv[5];
            P.q[0] = pv[6]; P.q[1] = pv[7]; P.q[2] = pv[8]; P.q[3] = pv[9];
            P.logit = pv[10];
        }
        float Yn[K];
        RecFields F{};
        float key = 0.0f;
        bool nvis = false;
        if constexpr (NEXT) {   // the geometry of project_store, its SH finiteness settled below
            ProjScalars S;
            project_scalars(P.means[0], P.means[1], P.means[2], P.ls[0], P.ls[1], P.ls[2], P.q[0], P.q[1], P.q[2],
                            P.q[3], P.logit, true, (double)alpha_min, S);
            const float fmx = P.means[0], fmy = P.means[1], fmz = P.means[2];
            Proj Pn;
            project_view(next_cam, fmx, fmy, fmz, fmx, fmy, fmz, P.q[0], P.q[1], P.q[2], P.q[3], S, depth_lo, depth_hi,
                         Pn);
            key = Pn.key;
            nvis = Pn.vis;
#pragma unroll
            for (int k = 0; k < K; ++k) Yn[k] = 0.0f;
            if (nvis) {
                sh_basis<DEG>(Pn.dir[0], Pn.dir[1], Pn.dir[2], Yn);
                F = rec_fields(Pn);
            }
        }
        load_pmv<kC>(0, i, shs, psh, msh, vsh);   // the first SH chunk (after the fp64 geometry: fewer live values)
        float Y[K];
        sh_basis<DEG>(dir[0], dir[1], dir[2], Y);
        float col[3] = {0.0f, 0.0f, 0.0f};
        bool fin = true;
#pragma unroll
        for (int c0 = 0; c0 < 3 * K; c0 += kC) {
            float pnx[kC], mnx[kC], vnx[kC];
            if (c0 + kC < 3 * K) load_pmv<kC>(c0 + kC, i, shs, pnx, mnx, vnx);   // the next chunk
            int cpl[kC];
            float gg[kC], sp[kC];
#pragma unroll
            for (int c = 0; c < kC; ++c) {
                const int plane = c0 + c;
                cpl[c] = plane;
                gg[c] = vis ? Y[plane / 3] * g.gc[plane % 3] : 0.0f;
                sp[c] = plane < 3 ? st[4] : st[5];
            }
            update(sgrp, cpl, gg, psh, sp, msh, vsh, i);
            if constexpr (NEXT) {
#pragma unroll
                for (int c = 0; c < kC; ++c) {
                    const int plane = c0 + c;
                    fin = fin && __builtin_isfinite(psh[c]);
                    col[plane % 3] = fmaf(psh[c], Yn[plane / 3], col[plane % 3]);
                }
            }
            if (c0 + kC < 3 * K) {
#pragma unroll
                for (int c = 0; c < kC; ++c) {
                    psh[c] = pnx[c];
                    msh[c] = mnx[c];
                    vsh[c] = vnx[c];
                }
            }
        }
        if constexpr (NEXT) {
            nvis = nvis && fin;   // a non-finite coefficient: culled, as project_view's scalars reject it
            next.depth[i] = key;
            next.radii[i] = nvis ? make_int2(F.rx, F.ry) : make_int2(0, 0);
            float4 rec[3];
            rec[0] = rec[1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            rec[2] = make_float4(0.0f, __uint_as_float((uint32_t)i), 0.0f, 0.0f);
            if (nvis) record_visible(F, col[0], col[1], col[2], i, next, rec);
            next.rec[3 * i + 0] = rec[0];
            next.rec[3 * i + 1] = rec[1];
            next.rec[3 * i + 2] = rec[2];
        }
    }

    // Chunk [c0, c0 + N) of the SH planes: parameter values (from the wave's LDS copy
    // shs[plane][lane]) and moments.
    template <int N>
    __device__ void load_pmv(int c0, int64_t i, float (*shs)[64], float (&pv)[N], float (&mv)[N],
                             float (&vv)[N]) const
    {
#pragma unroll
        for (int c = 0; c < N; ++c) {
            const int64_t idx = (int64_t)(c0 + c) * n + i;
            pv[c] = shs[c0 + c][threadIdx.x & 63];
            mv[c] = __builtin_nontemporal_load(m[4] + idx);
            vv[c] = __builtin_nontemporal_load(v[4] + idx);
        }
    }
};

// The colour's part of the chain rule through the view direction: d v^ = sum_k (sh_k . dc)
// grad Y_k, and its share of dL/dmu (dsh).
template <int DEG>
__device__ __forceinline__ void project_bwd_sh(const Proj &P, const float (&gc)[3], const float *shc, double (&dsh)[3])
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = shc[3 * k] * gc[0] + shc[3 * k + 1] * gc[1] + shc[3 * k + 2] * gc[2];
    float gx, gy, gz;
    sh_grad<DEG>(P.dir[0], P.dir[1], P.dir[2], wk, gx, gy, gz);
    const double vd = (double)P.dir[0] * gx + (double)P.dir[1] * gy + (double)P.dir[2] * gz;
    const double idist = 1.0 / P.dist;
    dsh[0] = (gx - P.dir[0] * vd) * idist;
    dsh[1] = (gy - P.dir[1] * vd) * idist;
    dsh[2] = (gz - P.dir[2] * vd) * idist;
}

// The chain rule for a Gaussian the projection keeps.  The colour's part comes first, so
// that the SH coefficients are no longer needed during the geometric part.
template <int DEG>
__device__ __forceinline__ void project_bwd_grads(const Proj &P, const CamD &cam, const float (&g2)[9],
                                                  const Params1<(DEG + 1) * (DEG + 1)> &prm,
                                                  Grad3<(DEG + 1) * (DEG + 1)> &G)
{
    const double gu = g2[0], gv = g2[1], gA = g2[2], gB = g2[3], gC = g2[4];
    const double go = g2[5];
    const float gc[3] = {g2[6], g2[7], g2[8]};
    double dsh[3];
    project_bwd_sh<DEG>(P, gc, prm.sh, dsh);

    // conic = Sigma2D^-1:  G_S2 = -Q G_Q Q with G_Q = [[gA, gB/2], [gB/2, gC]]
    const double A = P.A, B = P.B, C = P.C;
    const double hb = 0.5 * gB;
    const double p00 = A * gA + B * hb, p01 = A * hb + B * gC;
    const double p10 = B * gA + C * hb, p11 = B * hb + C * gC;
    const double s00 = -(p00 * A + p01 * B);
    const double s01 = -(p00 * B + p01 * C);
    const double s11 = -(p10 * B + p11 * C);

    // Sigma2D = T Sigma T^T:  G_T = 2 G_S2 T Sigma,  G_Sigma = T^T G_S2 T
    double R[9], M[9], S[6], T[6];
    rot_q(P.q[0], P.q[1], P.q[2], P.q[3], R);
    cov3d(R, P.s, M, S);
    jw(cam, P.X, P.Y, P.Z, T);
    double ts[6];
    for (int r = 0; r < 2; ++r) {
        const double *t = T + 3 * r;
        ts[3 * r + 0] = t[0] * S[0] + t[1] * S[1] + t[2] * S[2];
        ts[3 * r + 1] = t[0] * S[1] + t[1] * S[3] + t[2] * S[4];
        ts[3 * r + 2] = t[0] * S[2] + t[1] * S[4] + t[2] * S[5];
    }
    double GT[6];
    for (int c = 0; c < 3; ++c) {
        GT[c] = 2.0 * (s00 * ts[c] + s01 * ts[3 + c]);
        GT[3 + c] = 2.0 * (s01 * ts[c] + s11 * ts[3 + c]);
    }
    double gsT[6];   // G_S2 T
    for (int c = 0; c < 3; ++c) {
        gsT[c] = s00 * T[c] + s01 * T[3 + c];
        gsT[3 + c] = s01 * T[c] + s11 * T[3 + c];
    }
    double GS[9];
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) GS[3 * r + c] = T[r] * gsT[c] + T[3 + r] * gsT[3 + c];

    // T = J W:  G_J = G_T W^T; only J00, J02, J11, J12 are non-zero
    const double *W = cam.R;
    const double gj00 = GT[0] * W[0] + GT[1] * W[1] + GT[2] * W[2];
    const double gj02 = GT[0] * W[6] + GT[1] * W[7] + GT[2] * W[8];
    const double gj11 = GT[3] * W[3] + GT[4] * W[4] + GT[5] * W[5];
    const double gj12 = GT[3] * W[6] + GT[4] * W[7] + GT[5] * W[8];
    const double iz = 1.0 / P.Z, iz2 = iz * iz, iz3 = iz2 * iz;
    const double fx = cam.fx, fy = cam.fy, X = P.X, Yc = P.Y;
    const double dX = -gj02 * fx * iz2 + gu * fx * iz;
    const double dY = -gj12 * fy * iz2 + gv * fy * iz;
    const double dZ = -gj00 * fx * iz2 + gj02 * 2.0 * fx * X * iz3 - gj11 * fy * iz2 + gj12 * 2.0 * fy * Yc * iz3
                    - gu * fx * X * iz2 - gv * fy * Yc * iz2;
    double dmu[3];
    for (int j = 0; j < 3; ++j) dmu[j] = W[j] * dX + W[3 + j] * dY + W[6 + j] * dZ;

    // Sigma = M M^T: G_M = 2 G_Sigma M;  M = R diag(s)
    double GR[9];
    for (int k = 0; k < 3; ++k) {
        double ds = 0.0;
        for (int r = 0; r < 3; ++r) {
            const double gm = 2.0 * (GS[3 * r + 0] * M[k] + GS[3 * r + 1] * M[3 + k] + GS[3 * r + 2] * M[6 + k]);
            ds += gm * R[3 * r + k];
            GR[3 * r + k] = gm * P.s[k];
        }
        G.ls[k] = (float)(ds * P.s[k]);
    }
    // R(q^) -> q^ -> q
    const double w = P.q[0], x = P.q[1], y = P.q[2], z = P.q[3];
    double dq[4];
    dq[0] = 2.0 * (-z * GR[1] + y * GR[2] + z * GR[3] - x * GR[5] - y * GR[6] + x * GR[7]);
    dq[1] = 2.0 * (y * GR[1] + z * GR[2] + y * GR[3] - 2.0 * x * GR[4] - w * GR[5] + z * GR[6] + w * GR[7]
                   - 2.0 * x * GR[8]);
    dq[2] = 2.0 * (-2.0 * y * GR[0] + x * GR[1] + w * GR[2] + x * GR[3] + z * GR[5] - w * GR[6] + z * GR[7]
                   - 2.0 * y * GR[8]);
    dq[3] = 2.0 * (-2.0 * z * GR[0] - w * GR[1] + x * GR[2] + w * GR[3] - 2.0 * z * GR[4] + y * GR[5] + x * GR[6]
                   + y * GR[7]);
    const double qd = w * dq[0] + x * dq[1] + y * dq[2] + z * dq[3];
    const double iq = 1.0 / P.qnorm;
    for (int j = 0; j < 4; ++j) G.q[j] = (float)((dq[j] - P.q[j] * qd) * iq);

    G.logit = (float)(go * P.o * (1.0 - P.o));

    // colour: d sh_k = Y_k dc
    sh_basis<DEG>(P.dir[0], P.dir[1], P.dir[2], G.Y);
    G.gc[0] = gc[0]; G.gc[1] = gc[1]; G.gc[2] = gc[2];
    for (int j = 0; j < 3; ++j) G.means[j] = (float)(dmu[j] + dsh[j]);
}

// in: the screen-space gradients (u, v, A, B, C, o, r, g, b), or with RAW the per-Gaussian
// moment sums of the raster backward, turned into those gradients here with the record's
// conic and opacity as the forward pass rounded them (and stored to grads2d [9][n] if given).
// With NEXT (an AdamSink, which leaves the updated parameters in prm), the updated Gaussian
// is then projected for the next camera, exactly as gs_project would project it.
template <int DEG, bool RAW, bool NEXT, class Sink>
__device__ __forceinline__ void project_bwd_one(const float *__restrict__ means, const float *__restrict__ log_scales,
                                                const float *__restrict__ quats, const float *__restrict__ logits,
                                                const float *__restrict__ sh, int64_t n, int64_t ldp, int64_t i,
                                                const CamD &cam, float alpha_min, float depth_lo, float depth_hi,
                                                const float (&in)[9], float *__restrict__ grads2d, const Sink &out,
                                                const CamD &next_cam, const ProjOut &next)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    // A gradient sink needs no SH coefficients of a culled Gaussian (its gradients are zero):
    // they are loaded after the geometry has decided visibility, and non-finite ones cull
    // then, which gives the same result as checking them first.
    constexpr bool kLazySH = std::is_same<Sink, GradSink>::value && !NEXT;
    Params1<K> prm;
    if constexpr (kLazySH)
        load_geometry(means, log_scales, quats, logits, ldp, i, prm);
    else
        load_params<std::is_same<Sink, AdamSink>::value>(means, log_scales, quats, logits, sh, ldp, i, prm);
    const bool shf = kLazySH ? true : sh_finite(prm);
    Proj P;
    const float fmx = prm.means[0], fmy = prm.means[1], fmz = prm.means[2];
    project_core(cam, fmx, fmy, fmz, fmx, fmy, fmz, prm.ls[0], prm.ls[1], prm.ls[2], prm.q[0], prm.q[1], prm.q[2],
                 prm.q[3], prm.logit, shf, (double)alpha_min, depth_lo, depth_hi, P);
    if constexpr (kLazySH) {
        if (P.vis) {
            load_sh(sh, ldp, i, prm);
            if (!sh_finite(prm)) P.vis = false;
        }
    }
    // culled Gaussians get zero gradients; every lane reaches the one flush at the end, so
    // a wave issues the sink's memory traffic once
    Grad3<K> G;
    for (int j = 0; j < 3; ++j) G.means[j] = G.ls[j] = 0.0f;
    for (int j = 0; j < 4; ++j) G.q[j] = 0.0f;
    G.logit = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) G.Y[k] = 0.0f;
    G.gc[0] = G.gc[1] = G.gc[2] = 0.0f;
    if (RAW) {
        float g2[9];
        RecConic rc{0.0f, 0.0f, 0.0f, 0.0f};
        if (P.vis) rc = rec_conic(P);
        gsr::moments_to_grads(in, rc.a, rc.b, rc.c, rc.l, g2);
        if (grads2d) {
#pragma unroll
            for (int f = 0; f < 9; ++f) grads2d[(int64_t)f * n + i] = g2[f];
        }
        if (P.vis) project_bwd_grads<DEG>(P, cam, g2, prm, G);
    } else if (P.vis) {
        project_bwd_grads<DEG>(P, cam, in, prm, G);
    }
    out.flush(i, G, prm);
    if constexpr (NEXT) project_store<DEG>(prm, next_cam, alpha_min, depth_lo, depth_hi, i, next);
}

// k_grad_adam's Gaussian: the per-Gaussian moment sums in (as project_bwd_one with RAW; without
// RAW, the screen-space gradients themselves), the projection backward and
// AdamSink::flush_view.  The SH coefficients are kept in the wave's LDS (shs[plane][lane])
// from the load to the update, not in registers.
template <int DEG, bool NEXT, bool RAW = true>
__device__ __forceinline__ void grad_adam_one(const float *__restrict__ means, const float *__restrict__ log_scales,
                                              const float *__restrict__ quats, const float *__restrict__ logits,
                                              const float *__restrict__ sh, int64_t n, int64_t ldp, int64_t i,
                                              const CamD &cam, float alpha_min, float depth_lo, float depth_hi,
                                              const float (&in)[9], float *__restrict__ grads2d, const AdamSink &out,
                                              const CamD &next_cam, const ProjOut &next, float (*shs)[64])
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    const int lane = threadIdx.x & 63;
    Params1<K> prm;
    load_params<true>(means, log_scales, quats, logits, sh, ldp, i, prm);
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) shs[k][lane] = prm.sh[k];
    const bool shf = sh_finite(prm);
    Proj P;
    const float fmx = prm.means[0], fmy = prm.means[1], fmz = prm.means[2];
    project_core(cam, fmx, fmy, fmz, fmx, fmy, fmz, prm.ls[0], prm.ls[1], prm.ls[2], prm.q[0], prm.q[1], prm.q[2],
                 prm.q[3], prm.logit, shf, (double)alpha_min, depth_lo, depth_hi, P);
    Grad3<K> G;
    for (int j = 0; j < 3; ++j) G.means[j] = G.ls[j] = 0.0f;
    for (int j = 0; j < 4; ++j) G.q[j] = 0.0f;
    G.logit = 0.0f;
    G.gc[0] = G.gc[1] = G.gc[2] = 0.0f;
    float g2[9];
    if constexpr (RAW) {
        RecConic rc{0.0f, 0.0f, 0.0f, 0.0f};
        if (P.vis) rc = rec_conic(P);
        gsr::moments_to_grads(in, rc.a, rc.b, rc.c, rc.l, g2);
        if (grads2d) {
#pragma unroll
            for (int f = 0; f < 9; ++f) grads2d[(int64_t)f * n + i] = g2[f];
        }
    } else {
#pragma unroll
        for (int f = 0; f < 9; ++f) g2[f] = in[f];
    }
    float dir[3] = {0.0f, 0.0f, 1.0f};
    if (P.vis) {
        project_bwd_grads<DEG>(P, cam, g2, prm, G);
        dir[0] = P.dir[0]; dir[1] = P.dir[1]; dir[2] = P.dir[2];
    }
    out.flush_view<DEG, NEXT>(i, G, P.vis, dir, prm, shs, alpha_min, depth_lo, depth_hi, next_cam, next);
}

template <int DEG>
__global__ __launch_bounds__(256) void k_project_bwd(
    const float *__restrict__ means, const float *__restrict__ log_scales, const float *__restrict__ quats,
    const float *__restrict__ logits, const float *__restrict__ sh, int64_t n, int64_t ldp, CamD cam, float alpha_min,
    float depth_lo, float depth_hi, const float *__restrict__ g2, GradSink out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float g[9];
#pragma unroll
    for (int f = 0; f < 9; ++f) g[f] = g2[(int64_t)f * n + i];
    project_bwd_one<DEG, false, false>(means, log_scales, quats, logits, sh, n, ldp, i, cam, alpha_min, depth_lo,
                                       depth_hi, g, nullptr, out, cam, ProjOut{});
}

// The end of a training step per Gaussian: the per-Gaussian sum of Eq. 4 over its
// quadrant-record slots (as k_grad_reduce; optionally stored in grads2d), the projection
// backward, and the Adam update of every parameter scalar; with NEXT also the projection
// of the updated Gaussian for the next camera (into next).
// LDS of one wave of k_grad_adam: its slot-sum stage, then (once the sums are done) its
// lanes' SH coefficients between the projection backward and the update.
__host__ __device__ constexpr size_t grad_adam_wave_lds(int deg)
{
    const size_t shb = (size_t)3 * (deg + 1) * (deg + 1) * 64 * sizeof(float);
    return shb > sizeof(gsr::SlotStage) ? shb : sizeof(gsr::SlotStage);
}

template <int DEG, bool NEXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_grad_adam(
    const float *__restrict__ means, const float *__restrict__ log_scales, const float *__restrict__ quats,
    const float *__restrict__ logits, const float *__restrict__ sh, int64_t n, int64_t ldp, CamD cam, float alpha_min,
    float depth_lo, float depth_hi, const gsr::BinsHeader *__restrict__ hdr, const uint32_t *__restrict__ qoff,
    const float4 *__restrict__ qgrad, const uint32_t *__restrict__ qstamp, float *__restrict__ grads2d, AdamSink out,
    CamD next_cam, ProjOut next)
{
    extern __shared__ __align__(16) unsigned char ga_lds[];   // grad_adam_wave_lds(DEG) per wave
    unsigned char *wl = ga_lds + (threadIdx.x >> 6) * grad_adam_wave_lds(DEG);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float acc[9];
    gsr::raw_slot_sums(hdr, qoff, qgrad, qstamp, i, n, *reinterpret_cast<gsr::SlotStage *>(wl), acc);
    if (i >= n) return;
    // the wave's stage is no longer read (each wave reads only its own; the sums end with a
    // wave barrier): its bytes now hold the lanes' SH coefficients
    grad_adam_one<DEG, NEXT>(means, log_scales, quats, logits, sh, n, ldp, i, cam, alpha_min, depth_lo, depth_hi, acc,
                             grads2d, out, next_cam, next, reinterpret_cast<float(*)[64]>(wl));
}

// The owner's update from screen-space gradients already summed per Gaussian (g2 [9][n],
// e.g. decoded from other renderers' records): the projection backward, Adam and, with
// NEXT, the projection of the updated Gaussian for the next camera, per Gaussian in one
// pass, as k_grad_adam after its slot sums.
__host__ __device__ constexpr size_t proj_bwd_adam_wave_lds(int deg)
{
    return (size_t)3 * (deg + 1) * (deg + 1) * 64 * sizeof(float);
}

template <int DEG, bool NEXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_proj_bwd_adam(
    const float *__restrict__ means, const float *__restrict__ log_scales, const float *__restrict__ quats,
    const float *__restrict__ logits, const float *__restrict__ sh, int64_t n, int64_t ldp, CamD cam, float alpha_min,
    float depth_lo, float depth_hi, const float *__restrict__ g2, AdamSink out, CamD next_cam, ProjOut next)
{
    extern __shared__ __align__(16) unsigned char pba_lds[];   // proj_bwd_adam_wave_lds(DEG) per wave
    float(*shs)[64] = reinterpret_cast<float(*)[64]>(pba_lds + (threadIdx.x >> 6) * proj_bwd_adam_wave_lds(DEG));
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float g[9];
#pragma unroll
    for (int f = 0; f < 9; ++f) g[f] = __builtin_nontemporal_load(g2 + (int64_t)f * n + i);
    grad_adam_one<DEG, NEXT, false>(means, log_scales, quats, logits, sh, n, ldp, i, cam, alpha_min, depth_lo,
                                    depth_hi, g, nullptr, out, next_cam, next, shs);
}

// -------------------------------------------------------------------- batches of views
// A training step over a batch of views (ROCm blog, "Batching and Hyperparameter Scaling":
// several camera views per optimiser step): the Gaussians are projected for every view of
// the batch in one pass over the parameters, each view is binned and rasterized on its own,
// and one pass per Gaussian sums each view's slots, takes each view's projection backward,
// adds the 3D gradients over the views, applies one Adam update and projects the updated
// Gaussian for the views of the next batch.
constexpr int kMaxViews = 4;

struct ViewBins {
    const gsr::BinsHeader *hdr;
    const uint32_t *qoff;
    const float4 *qgrad;
    const uint32_t *qstamp;
};

struct BatchProj {
    int views;
    CamD cam[kMaxViews];
    ProjOut out[kMaxViews];
};

struct BatchGrad {
    int views;
    float grad_scale;
    CamD cam[kMaxViews];
    ViewBins vb[kMaxViews];
};

// 3D gradients summed over views; the SH gradients as per-plane sums of Y_k(v^) dL/dc,
// kept in LDS (one column per thread of the block) to leave the registers to the
// projection backward.
template <int K>
struct GradSum {
    float means[3], ls[3], q[4], logit;
    float (*shg)[256];
    int t;
    __device__ float sh(int plane) const { return shg[plane][t]; }
};

template <int DEG>
__global__ __launch_bounds__(256) void k_project_batch(const float *__restrict__ means,
                                                       const float *__restrict__ log_scales,
                                                       const float *__restrict__ quats, const float *__restrict__ logits,
                                                       const float *__restrict__ sh, int64_t n, int64_t ldp,
                                                       float alpha_min, float depth_lo, float depth_hi, BatchProj bp)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    Params1<K> prm;
    load_params<false>(means, log_scales, quats, logits, sh, ldp, i, prm);
    ProjScalars S;
    params_scalars(prm, alpha_min, S);
    for (int v = 0; v < bp.views; ++v) project_store_s<DEG>(prm, S, bp.cam[v], depth_lo, depth_hi, i, bp.out[v]);
}

// Per Gaussian: for each view in order, the Eq. 4 sum over that view's slots, scaled by
// grad_scale (the batch mean: 1 / views), and the projection backward for that view's
// camera, added to the running 3D gradients; then the Adam update; with NEXT, the
// projections of the updated Gaussian for the next batch's views.
template <int DEG, bool NEXT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_grad_adam_batch(
    const float *__restrict__ means, const float *__restrict__ log_scales, const float *__restrict__ quats,
    const float *__restrict__ logits, const float *__restrict__ sh, int64_t n, int64_t ldp, float alpha_min,
    float depth_lo, float depth_hi, BatchGrad bg, AdamSink out, BatchProj next)
{
    constexpr int K = (DEG + 1) * (DEG + 1);
    __shared__ gsr::SlotStage stage[4];
    __shared__ float shacc[3 * K][256];
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = i < n;
    Params1<K> prm;
    ProjScalars PS;
    PS.ok = false;
    if (live) {
        load_params<true>(means, log_scales, quats, logits, sh, ldp, i, prm);
        params_scalars(prm, alpha_min, PS);
    }
    GradSum<K> S;
    for (int j = 0; j < 3; ++j) S.means[j] = S.ls[j] = 0.0f;
    for (int j = 0; j < 4; ++j) S.q[j] = 0.0f;
    S.logit = 0.0f;
    S.shg = shacc;
    S.t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 3 * K; ++k) shacc[k][threadIdx.x] = 0.0f;
    for (int v = 0; v < bg.views; ++v) {
        float acc[9];
        // every lane of the wave takes part in the slot sums
        gsr::raw_slot_sums<2>(bg.vb[v].hdr, bg.vb[v].qoff, bg.vb[v].qgrad, bg.vb[v].qstamp, i, n,
                           stage[threadIdx.x >> 6], acc);
        if (live) {
            Proj P;
            const float fmx = prm.means[0], fmy = prm.means[1], fmz = prm.means[2];
            project_view(bg.cam[v], fmx, fmy, fmz, fmx, fmy, fmz, prm.q[0], prm.q[1], prm.q[2], prm.q[3], PS, depth_lo,
                         depth_hi, P);
            if (P.vis) {
                const RecConic rc = rec_conic(P);
                float g2[9];
                gsr::moments_to_grads(acc, rc.a, rc.b, rc.c, rc.l, g2);
#pragma unroll
                for (int f = 0; f < 9; ++f) g2[f] *= bg.grad_scale;
                Grad3<K> G;
                project_bwd_grads<DEG>(P, bg.cam[v], g2, prm, G);
                for (int j = 0; j < 3; ++j) { S.means[j] += G.means[j]; S.ls[j] += G.ls[j]; }
                for (int j = 0; j < 4; ++j) S.q[j] += G.q[j];
                S.logit += G.logit;
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int c = 0; c < 3; ++c) shacc[3 * k + c][threadIdx.x] += G.Y[k] * G.gc[c];
            }
        }
    }
    if (!live) return;
    out.flush(i, S, prm);
    if constexpr (NEXT) {
        params_scalars(prm, alpha_min, PS);   // of the updated Gaussian
        for (int v = 0; v < next.views; ++v)
            project_store_s<DEG>(prm, PS, next.cam[v], depth_lo, depth_hi, i, next.out[v]);
    }
}

}  // namespace

namespace gsi {

gs_status check_gaussians(const gs_gaussians *g)
{
    if (!g) return fail(GS_ERR_INVALID_ARGUMENT, "gaussians is NULL");
    if (g->n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
    if (g->n > (int64_t(1) << 31) - 1) return fail(GS_ERR_UNSUPPORTED, "n >= 2^31");
    if (g->n > 0 && (!g->means || !g->log_scales || !g->quats || !g->opacity_logits || !g->sh))
        return fail(GS_ERR_INVALID_ARGUMENT, "a parameter pointer is NULL");
    if (g->ld != 0 && g->ld < g->n) return fail(GS_ERR_INVALID_ARGUMENT, "plane stride ld < n");
    return GS_OK;
}

gs_status check_proj_out(const gs_projected *out, int64_t n)
{
    if (!out) return fail(GS_ERR_INVALID_ARGUMENT, "projected output is NULL");
    if (n == 0) return GS_OK;
    if (!out->depth || !out->radii || !out->rec)
        return fail(GS_ERR_INVALID_ARGUMENT, "projected depth / radii / rec is NULL");
    if (!aligned(out->rec, 16) || !aligned(out->radii, 8))
        return fail(GS_ERR_INVALID_ARGUMENT, "rec must be 16-byte, radii 8-byte aligned");
    return GS_OK;
}

ProjOut proj_out(const gs_projected *out, int64_t n)
{
    return ProjOut{out->means2d, out->conic_opacity, out->color, out->depth, reinterpret_cast<int2 *>(out->radii),
                   reinterpret_cast<float4 *>(out->rec), n};
}

gs_status launch_project_bwd(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                             const float *grads2d, gs_param_grads *out, hipStream_t stream)
{
    const int64_t n = g->n;
    if (n == 0) return GS_OK;
    if (!out->means || !out->log_scales || !out->quats || !out->opacity_logits || !out->sh)
        return fail(GS_ERR_INVALID_ARGUMENT, "a grads3d pointer is NULL");
    if (out->ld != 0 && out->ld < n) return fail(GS_ERR_INVALID_ARGUMENT, "grads3d plane stride ld < n");
    const CamD cd = make_cam(cam);
    const dim3 grid((unsigned)ceil_div(n, 256)), block(256);
    const GradSink sink{out->means, out->log_scales, out->quats, out->opacity_logits, out->sh, grads_ld(out, n)};
#define GS_PB(D)                                                                                              \
    k_project_bwd<D><<<grid, block, 0, stream>>>(g->means, g->log_scales, g->quats, g->opacity_logits, g->sh, \
                                                 n, param_ld(g), cd, p->alpha_min, p->depth_lo, p->depth_hi,   \
                                                 grads2d, sink)
    switch (p->sh_degree) {
    case 0: GS_PB(0); break;
    case 1: GS_PB(1); break;
    case 2: GS_PB(2); break;
    default: GS_PB(3); break;
    }
#undef GS_PB
    GS_LAUNCH_CHECK("k_project_bwd");
    return GS_OK;
}

}  // namespace gsi

extern "C" gs_status gs_project(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                                gs_projected *out, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    const int64_t n = g->n;
    if ((s = check_proj_out(out, n)) != GS_OK) return s;
    if (n == 0) return GS_OK;
    const CamD cd = make_cam(cam);
    const dim3 grid((unsigned)ceil_div(n, 256)), block(256);
    const ProjOut po = proj_out(out, n);
#define GS_PF(D)                                                                                        \
    k_project<D><<<grid, block, 0, stream>>>(g->means, g->log_scales, g->quats, g->opacity_logits, g->sh, n, \
                                             param_ld(g), cd, p->alpha_min, p->depth_lo, p->depth_hi, po)
    switch (p->sh_degree) {
    case 0: GS_PF(0); break;
    case 1: GS_PF(1); break;
    case 2: GS_PF(2); break;
    default: GS_PF(3); break;
    }
#undef GS_PF
    GS_LAUNCH_CHECK("k_project");
    return GS_OK;
}

extern "C" gs_status gs_project_bwd(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                                    const float *grads2d, gs_param_grads *grads3d, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if (!grads3d) return fail(GS_ERR_INVALID_ARGUMENT, "grads3d is NULL");
    if (g->n > 0 && !grads2d) return fail(GS_ERR_INVALID_ARGUMENT, "grads2d is NULL");
    return launch_project_bwd(g, cam, p, grads2d, grads3d, stream);
}

namespace gsi {
gs_status check_raster_inputs(const gs_bins *bins, const gs_camera *cam);
}

namespace {

gs_status make_adam_sink(const gs_gaussians *g, const gs_param_grads *m, const gs_param_grads *v,
                         const gs_adam_lrs *lr, int32_t step, float beta1, float beta2, float eps, AdamSink &sink)
{
    using namespace gsi;
    if (!m->means || !m->log_scales || !m->quats || !m->opacity_logits || !m->sh || !v->means || !v->log_scales ||
        !v->quats || !v->opacity_logits || !v->sh)
        return fail(GS_ERR_INVALID_ARGUMENT, "an Adam moment pointer is NULL");
    float *params[5] = {const_cast<float *>(g->means), const_cast<float *>(g->log_scales), const_cast<float *>(g->quats),
                        const_cast<float *>(g->opacity_logits), const_cast<float *>(g->sh)};
    float *ms[5] = {m->means, m->log_scales, m->quats, m->opacity_logits, m->sh};
    float *vs[5] = {v->means, v->log_scales, v->quats, v->opacity_logits, v->sh};
    for (int a = 0; a < 5; ++a) { sink.p[a] = params[a]; sink.m[a] = ms[a]; sink.v[a] = vs[a]; }
    // p, m and v share one plane stride
    const int64_t ld = param_ld(g);
    if (grads_ld(m, g->n) != ld || grads_ld(v, g->n) != ld)
        return fail(GS_ERR_INVALID_ARGUMENT, "the Adam moments must have the parameters' plane stride");
    sink.n = ld;
    // the same host arithmetic as gs_adam_step, so that both paths agree bit for bit
    const double bc1 = 1.0 - std::pow((double)beta1, step), bc2 = 1.0 - std::pow((double)beta2, step);
    const float lrs[6] = {lr->means, lr->log_scales, lr->quats, lr->opacity_logits, lr->sh_dc, lr->sh_rest};
    for (int a = 0; a < 6; ++a) sink.st[a] = (float)((double)lrs[a] / bc1);
    sink.b1 = beta1;
    sink.b2 = beta2;
    sink.inv_bc2 = (float)(1.0 / bc2);
    sink.eps = eps;
    return GS_OK;
}

gs_status check_adam_args(const gs_param_grads *m, const gs_param_grads *v, const gs_adam_lrs *lr, int32_t step,
                          float beta1, float beta2, float eps)
{
    using namespace gsi;
    if (!m || !v || !lr) return fail(GS_ERR_INVALID_ARGUMENT, "m / v / lr is NULL");
    if (step < 1) return fail(GS_ERR_INVALID_ARGUMENT, "step must be >= 1");
    if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f && eps >= 0.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "bad Adam hyper-parameters");
    return GS_OK;
}

ViewBins view_bins(const gs_bins *bins, const gs_camera *cam, int64_t n)
{
    const int T = gsi::tiles_x(cam->width) * gsi::tiles_y(cam->height);
    const gsr::RasterLayout L = gsr::raster_layout(n, bins->capacity, T);
    const char *rb = static_cast<const char *>(bins->raster);
    return ViewBins{reinterpret_cast<const gsr::BinsHeader *>(rb + L.hdr),
                    reinterpret_cast<const uint32_t *>(rb + L.qoff), reinterpret_cast<const float4 *>(rb + L.qgrad),
                    reinterpret_cast<const uint32_t *>(rb + L.qstamp)};
}

gs_status grad_adam_launch(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins, const gs_camera *cam,
                           const gs_raster_params *p, float *grads2d, const gs_param_grads *m,
                           const gs_param_grads *v, const gs_adam_lrs *lr, int32_t step, float beta1, float beta2,
                           float eps, const gs_camera *next_cam, gs_projected *next_proj, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_raster_inputs(bins, cam)) != GS_OK) return s;
    if (!m || !v || !lr) return fail(GS_ERR_INVALID_ARGUMENT, "m / v / lr is NULL");
    if (g->n > 0 && (!proj || !proj->rec || !aligned(proj->rec, 16)))
        return fail(GS_ERR_INVALID_ARGUMENT, "proj->rec is NULL or not 16-byte aligned");
    if (step < 1) return fail(GS_ERR_INVALID_ARGUMENT, "step must be >= 1");
    if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f && eps >= 0.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "bad Adam hyper-parameters");
    const int64_t n = g->n;
    if (next_cam) {
        if ((s = check_camera(next_cam)) != GS_OK) return s;
        if ((s = check_proj_out(next_proj, n)) != GS_OK) return s;
    }
    if (n == 0) return GS_OK;
    AdamSink sink;
    if ((s = make_adam_sink(g, m, v, lr, step, beta1, beta2, eps, sink)) != GS_OK) return s;
    const int T = tiles_x(cam->width) * tiles_y(cam->height);
    const gsr::RasterLayout L = gsr::raster_layout(n, bins->capacity, T);
    const char *rb = static_cast<const char *>(bins->raster);
    const gsr::BinsHeader *hdr = reinterpret_cast<const gsr::BinsHeader *>(rb + L.hdr);
    const uint32_t *qoff = reinterpret_cast<const uint32_t *>(rb + L.qoff);
    const float4 *qg = reinterpret_cast<const float4 *>(rb + L.qgrad);
    const uint32_t *qs = reinterpret_cast<const uint32_t *>(rb + L.qstamp);
    const CamD cd = make_cam(cam);
    const CamD nd = next_cam ? make_cam(next_cam) : cd;
    const ProjOut po = next_cam ? proj_out(next_proj, n) : ProjOut{};
    // Small blocks: at two waves per SIMD the last round of blocks is the coarser the larger
    // they are.  Measured on MI355X: 64 threads fastest at 1M Gaussians, 128 at 10M.
    const int bt = n <= (int64_t(1) << 22) ? 64 : 128;
    const dim3 grid((unsigned)ceil_div(n, (int64_t)bt)), block((unsigned)bt);
#define GS_GA(D)                                                                                                   \
    do {                                                                                                           \
        const size_t lds = (size_t)(bt / 64) * grad_adam_wave_lds(D);                                              \
        if (next_cam)                                                                                              \
            k_grad_adam<D, true><<<grid, block, lds, stream>>>(g->means, g->log_scales, g->quats,                  \
                                                               g->opacity_logits, g->sh, n, param_ld(g), cd,       \
                                                               p->alpha_min, p->depth_lo, p->depth_hi, hdr, qoff,  \
                                                               qg, qs, grads2d, sink, nd, po);                     \
        else                                                                                                       \
            k_grad_adam<D, false><<<grid, block, lds, stream>>>(g->means, g->log_scales, g->quats,                 \
                                                                g->opacity_logits, g->sh, n, param_ld(g), cd,      \
                                                                p->alpha_min, p->depth_lo, p->depth_hi, hdr, qoff, \
                                                                qg, qs, grads2d, sink, nd, po);                    \
    } while (0)
    switch (p->sh_degree) {
    case 0: GS_GA(0); break;
    case 1: GS_GA(1); break;
    case 2: GS_GA(2); break;
    default: GS_GA(3); break;
    }
#undef GS_GA
    GS_LAUNCH_CHECK("k_grad_adam");
    return GS_OK;
}

}  // namespace

extern "C" gs_status gs_grad_aggregate_adam(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                                            const gs_camera *cam, const gs_raster_params *p, float *grads2d,
                                            const gs_param_grads *m, const gs_param_grads *v, const gs_adam_lrs *lr,
                                            int32_t step, float beta1, float beta2, float eps, hipStream_t stream)
{
    return grad_adam_launch(g, proj, bins, cam, p, grads2d, m, v, lr, step, beta1, beta2, eps, nullptr, nullptr,
                            stream);
}

extern "C" gs_status gs_grad_aggregate_adam_project(const gs_gaussians *g, const gs_projected *proj,
                                                    const gs_bins *bins, const gs_camera *cam,
                                                    const gs_raster_params *p, float *grads2d,
                                                    const gs_param_grads *m, const gs_param_grads *v,
                                                    const gs_adam_lrs *lr, int32_t step, float beta1, float beta2,
                                                    float eps, const gs_camera *next_cam, gs_projected *next_proj,
                                                    hipStream_t stream)
{
    if (!next_cam) return gsi::fail(GS_ERR_INVALID_ARGUMENT, "next_cam is NULL");
    return grad_adam_launch(g, proj, bins, cam, p, grads2d, m, v, lr, step, beta1, beta2, eps, next_cam, next_proj,
                            stream);
}

extern "C" gs_status gs_project_bwd_adam(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                                        const float *grads2d, const gs_param_grads *m, const gs_param_grads *v,
                                        const gs_adam_lrs *lr, int32_t step, float beta1, float beta2, float eps,
                                        const gs_camera *next_cam, gs_projected *next_proj, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_camera(cam)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_adam_args(m, v, lr, step, beta1, beta2, eps)) != GS_OK) return s;
    const int64_t n = g->n;
    if (n > 0 && !grads2d) return fail(GS_ERR_INVALID_ARGUMENT, "grads2d is NULL");
    if (next_cam) {
        if ((s = check_camera(next_cam)) != GS_OK) return s;
        if ((s = check_proj_out(next_proj, n)) != GS_OK) return s;
    }
    if (n == 0) return GS_OK;
    AdamSink sink;
    if ((s = make_adam_sink(g, m, v, lr, step, beta1, beta2, eps, sink)) != GS_OK) return s;
    const CamD cd = make_cam(cam);
    const CamD nd = next_cam ? make_cam(next_cam) : cd;
    const ProjOut po = next_cam ? proj_out(next_proj, n) : ProjOut{};
    const int bt = n <= (int64_t(1) << 22) ? 64 : 128;   // as k_grad_adam
    const dim3 grid((unsigned)ceil_div(n, (int64_t)bt)), block((unsigned)bt);
#define GS_PBA(D)                                                                                                  \
    do {                                                                                                           \
        const size_t lds = (size_t)(bt / 64) * proj_bwd_adam_wave_lds(D);                                          \
        if (next_cam)                                                                                              \
            k_proj_bwd_adam<D, true><<<grid, block, lds, stream>>>(g->means, g->log_scales, g->quats,              \
                                                                   g->opacity_logits, g->sh, n, param_ld(g), cd,   \
                                                                   p->alpha_min, p->depth_lo, p->depth_hi, grads2d, \
                                                                   sink, nd, po);                                  \
        else                                                                                                       \
            k_proj_bwd_adam<D, false><<<grid, block, lds, stream>>>(g->means, g->log_scales, g->quats,             \
                                                                    g->opacity_logits, g->sh, n, param_ld(g), cd,  \
                                                                    p->alpha_min, p->depth_lo, p->depth_hi,        \
                                                                    grads2d, sink, nd, po);                        \
    } while (0)
    switch (p->sh_degree) {
    case 0: GS_PBA(0); break;
    case 1: GS_PBA(1); break;
    case 2: GS_PBA(2); break;
    default: GS_PBA(3); break;
    }
#undef GS_PBA
    GS_LAUNCH_CHECK("k_proj_bwd_adam");
    return GS_OK;
}

extern "C" gs_status gs_project_batch(const gs_gaussians *g, int32_t views, const gs_camera *cams,
                                      const gs_raster_params *p, gs_projected *out, hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if (views < 1 || views > kMaxViews) return fail(GS_ERR_INVALID_ARGUMENT, "views must lie in [1, %d]", kMaxViews);
    if (!cams || !out) return fail(GS_ERR_INVALID_ARGUMENT, "cams / out is NULL");
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    BatchProj bp = {};
    bp.views = views;
    for (int v = 0; v < views; ++v) {
        if ((s = check_camera(&cams[v])) != GS_OK) return s;
        if ((s = check_proj_out(&out[v], g->n)) != GS_OK) return s;
        bp.cam[v] = make_cam(&cams[v]);
        bp.out[v] = proj_out(&out[v], g->n);
    }
    const int64_t n = g->n;
    if (n == 0) return GS_OK;
    const dim3 grid((unsigned)ceil_div(n, 256)), block(256);
#define GS_PB(D)                                                                                                    \
    k_project_batch<D><<<grid, block, 0, stream>>>(g->means, g->log_scales, g->quats, g->opacity_logits, g->sh, n, \
                                                   param_ld(g), p->alpha_min, p->depth_lo, p->depth_hi, bp)
    switch (p->sh_degree) {
    case 0: GS_PB(0); break;
    case 1: GS_PB(1); break;
    case 2: GS_PB(2); break;
    default: GS_PB(3); break;
    }
#undef GS_PB
    GS_LAUNCH_CHECK("k_project_batch");
    return GS_OK;
}

extern "C" gs_status gs_grad_aggregate_adam_batch(const gs_gaussians *g, int32_t views, const gs_bins *bins,
                                                  const gs_camera *cams, const gs_raster_params *p, float grad_scale,
                                                  const gs_param_grads *m, const gs_param_grads *v,
                                                  const gs_adam_lrs *lr, int32_t step, float beta1, float beta2,
                                                  float eps, const gs_camera *next_cams, gs_projected *next_proj,
                                                  hipStream_t stream)
{
    using namespace gsi;
    gs_status s;
    if (views < 1 || views > kMaxViews) return fail(GS_ERR_INVALID_ARGUMENT, "views must lie in [1, %d]", kMaxViews);
    if (!bins || !cams) return fail(GS_ERR_INVALID_ARGUMENT, "bins / cams is NULL");
    if ((s = check_gaussians(g)) != GS_OK) return s;
    if ((s = check_params(p)) != GS_OK) return s;
    if ((s = check_adam_args(m, v, lr, step, beta1, beta2, eps)) != GS_OK) return s;
    if (!(grad_scale > 0.0f) || !__builtin_isfinite(grad_scale))
        return fail(GS_ERR_INVALID_ARGUMENT, "grad_scale must be positive and finite");
    const int64_t n = g->n;
    BatchGrad bg = {};
    bg.views = views;
    bg.grad_scale = grad_scale;
    for (int k = 0; k < views; ++k) {
        if ((s = check_camera(&cams[k])) != GS_OK) return s;
        if ((s = check_raster_inputs(&bins[k], &cams[k])) != GS_OK) return s;
        bg.cam[k] = make_cam(&cams[k]);
        bg.vb[k] = view_bins(&bins[k], &cams[k], n);
    }
    BatchProj next = {};
    if (next_cams) {
        if (!next_proj) return fail(GS_ERR_INVALID_ARGUMENT, "next_proj is NULL");
        next.views = views;
        for (int k = 0; k < views; ++k) {
            if ((s = check_camera(&next_cams[k])) != GS_OK) return s;
            if ((s = check_proj_out(&next_proj[k], n)) != GS_OK) return s;
            next.cam[k] = make_cam(&next_cams[k]);
            next.out[k] = proj_out(&next_proj[k], n);
        }
    }
    if (n == 0) return GS_OK;
    AdamSink sink;
    if ((s = make_adam_sink(g, m, v, lr, step, beta1, beta2, eps, sink)) != GS_OK) return s;
    const dim3 grid((unsigned)ceil_div(n, 256)), block(256);
#define GS_GB(D)                                                                                                     \
    do {                                                                                                             \
        if (next_cams)                                                                                               \
            k_grad_adam_batch<D, true><<<grid, block, 0, stream>>>(g->means, g->log_scales, g->quats,                \
                                                                   g->opacity_logits, g->sh, n, param_ld(g),         \
                                                                   p->alpha_min, p->depth_lo, p->depth_hi, bg, sink, \
                                                                   next);                                            \
        else                                                                                                         \
            k_grad_adam_batch<D, false><<<grid, block, 0, stream>>>(g->means, g->log_scales, g->quats,               \
                                                                    g->opacity_logits, g->sh, n, param_ld(g),        \
                                                                    p->alpha_min, p->depth_lo, p->depth_hi, bg,      \
                                                                    sink, next);                                     \
    } while (0)
    switch (p->sh_degree) {
    case 0: GS_GB(0); break;
    case 1: GS_GB(1); break;
    case 2: GS_GB(2); break;
    default: GS_GB(3); break;
    }
#undef GS_GB
    GS_LAUNCH_CHECK("k_grad_adam_batch");
    return GS_OK;
}
