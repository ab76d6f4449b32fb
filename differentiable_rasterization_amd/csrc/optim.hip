// L1 loss and Adam.
//
// Loss: the L1 term of the objective (ByteSplat, section 2.1, Eq. 2; "Scaling 3D
// Gaussian Splatting with Distributed Compute", loss of section "Why gsplat Cannot
// Just Use DDP"), as the mean over all colour values, and its gradient.
// Adam: textbook bias-corrected Adam with the settings of that page's
// create_splats_with_optimizers excerpt at batch size 1 (eps 1e-15, betas 0.9 / 0.999).
// Both kernels are pure HBM streams: float4 loads and stores, grid-stride loops.
#include <cmath>

#include "kernels.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_loss_l1(const float *__restrict__ c, const float *__restrict__ t,
                                                      int64_t m, float inv, float *__restrict__ grad,
                                                      double *__restrict__ partials)
{
    __shared__ double red[kThreads / 64];
    double acc = 0.0;
    const int64_t m4 = m / 4;
    const float4 *c4 = reinterpret_cast<const float4 *>(c);
    const float4 *t4 = reinterpret_cast<const float4 *>(t);
    float4 *g4 = reinterpret_cast<float4 *>(grad);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    auto sgn = [](float d) { return d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f); };
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < m4; i += stride) {
        const float4 a = c4[i], b = t4[i];
        const float d0 = a.x - b.x, d1 = a.y - b.y, d2 = a.z - b.z, d3 = a.w - b.w;
        acc += (double)(fabsf(d0) + fabsf(d1)) + (double)(fabsf(d2) + fabsf(d3));
        g4[i] = make_float4(sgn(d0) * inv, sgn(d1) * inv, sgn(d2) * inv, sgn(d3) * inv);
    }
    for (int64_t i = 4 * m4 + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < m; i += stride) {
        const float d = c[i] - t[i];
        acc += (double)fabsf(d);
        grad[i] = sgn(d) * inv;
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_down(acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) partials[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kThreads) void k_loss_final(const double *__restrict__ partials, int nb, double inv,
                                                         float *__restrict__ loss)
{
    __shared__ double red[kThreads / 64];
    double acc = 0.0;
    for (int i = threadIdx.x; i < nb; i += kThreads) acc += partials[i];
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_down(acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) *loss = (float)((red[0] + red[1] + red[2] + red[3]) * inv);
}

constexpr int kMaxGroups = 16;

typedef float v4f __attribute__((ext_vector_type(4)));

struct AdamArgs {
    float *p[kMaxGroups];
    const float *g[kMaxGroups];
    float *m[kMaxGroups];
    float *v[kMaxGroups];
    int64_t n[kMaxGroups];
    uint32_t block0[kMaxGroups + 1];   // first block of each group
    float step[kMaxGroups];            // lr / (1 - b1^t)
    int32_t head[kMaxGroups];          // vector groups: scalars before the first 16-byte boundary
    bool vec[kMaxGroups];              // the four arrays share their offset from a 16-byte boundary
    int ng;
    float b1, b2, inv_bc2, eps;
};

using gsd::adam_update;

__device__ __forceinline__ void adam_scalar(const AdamArgs &a, int gi, int64_t e)
{
    float p = a.p[gi][e], m = a.m[gi][e], v = a.v[gi][e];
    adam_update(p, a.g[gi][e], m, v, a.b1, a.b2, a.inv_bc2, a.eps, a.step[gi]);
    a.p[gi][e] = p;
    a.m[gi][e] = m;
    a.v[gi][e] = v;
}

// Vector groups: one float4 of the group's aligned body per thread, plus the up to three
// scalars before and after the body in the group's first block.  Other groups: one scalar
// per thread.  Every block lies inside one group.  The four streams are read and written
// once, so the accesses are non-temporal (they would only evict other data from the caches).
__global__ __launch_bounds__(kThreads) void k_adam(AdamArgs a)
{
    const uint32_t b = blockIdx.x;
    int gi = 0;
    while (gi + 1 < a.ng && b >= a.block0[gi + 1]) ++gi;
    const int64_t lb = b - a.block0[gi];
    const int64_t n = a.n[gi];
    if (!a.vec[gi]) {
        const int64_t e = lb * kThreads + threadIdx.x;
        if (e < n) adam_scalar(a, gi, e);
        return;
    }
    const int64_t head = a.head[gi];
    const int64_t n4 = (n - head) >> 2;
    const int64_t j = lb * kThreads + threadIdx.x;   // float4 index in the body
    if (lb == 0) {
        const int64_t tail = n - head - 4 * n4;
        if ((int64_t)threadIdx.x < head) adam_scalar(a, gi, threadIdx.x);
        if (threadIdx.x >= 64 && (int64_t)threadIdx.x < 64 + tail) adam_scalar(a, gi, head + 4 * n4 + threadIdx.x - 64);
    }
    if (j >= n4) return;
    const float st = a.step[gi];
    v4f *pp = reinterpret_cast<v4f *>(a.p[gi] + head) + j;
    const v4f *gp = reinterpret_cast<const v4f *>(a.g[gi] + head) + j;
    v4f *mp = reinterpret_cast<v4f *>(a.m[gi] + head) + j;
    v4f *vp = reinterpret_cast<v4f *>(a.v[gi] + head) + j;
    v4f p = __builtin_nontemporal_load(pp), g = __builtin_nontemporal_load(gp);
    v4f m = __builtin_nontemporal_load(mp), v = __builtin_nontemporal_load(vp);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float pc = p[c], mc = m[c], vc = v[c];
        adam_update(pc, g[c], mc, vc, a.b1, a.b2, a.inv_bc2, a.eps, st);
        p[c] = pc;
        m[c] = mc;
        v[c] = vc;
    }
    __builtin_nontemporal_store(p, pp);
    __builtin_nontemporal_store(m, mp);
    __builtin_nontemporal_store(v, vp);
}

int stream_blocks(int64_t work)
{
    // enough blocks to fill 256 CUs several times over, grid-stride beyond that
    const int64_t b = gsi::ceil_div(work, kThreads);
    return (int)std::min<int64_t>(std::max<int64_t>(b, 1), 256 * 16);
}

}  // namespace

extern "C" size_t gs_loss_workspace_bytes(int64_t n_px)
{
    (void)n_px;
    return sizeof(double) * 256 * 16;
}

extern "C" gs_status gs_loss_l1(const float *color, const float *target, int64_t n_px, float *loss_out,
                                float *dL_dcolor, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    using namespace gsi;
    if (n_px < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n_px < 0");
    if (n_px == 0) {
        if (loss_out) return fill_f32(loss_out, 1, 0.0f, stream);
        return GS_OK;
    }
    if (!color || !target || !dL_dcolor) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(color, 16) || !aligned(target, 16) || !aligned(dL_dcolor, 16))
        return fail(GS_ERR_INVALID_ARGUMENT, "color / target / dL_dcolor must be 16-byte aligned");
    if (!workspace || workspace_bytes < gs_loss_workspace_bytes(n_px) || !aligned(workspace, 8))
        return fail(GS_ERR_INVALID_ARGUMENT, "workspace too small");
    const int64_t m = 3 * n_px;
    const int nb = stream_blocks(m / 4 + 1);
    double *part = static_cast<double *>(workspace);
    k_loss_l1<<<nb, kThreads, 0, stream>>>(color, target, m, (float)(1.0 / (double)m), dL_dcolor, part);
    GS_LAUNCH_CHECK("k_loss_l1");
    if (loss_out) {
        k_loss_final<<<1, kThreads, 0, stream>>>(part, nb, 1.0 / (double)m, loss_out);
        GS_LAUNCH_CHECK("k_loss_final");
    }
    return GS_OK;
}

extern "C" gs_status gs_adam_step(const gs_adam_group *groups, int32_t n_groups, int32_t step, float beta1,
                                  float beta2, float eps, hipStream_t stream)
{
    using namespace gsi;
    if (n_groups < 0 || n_groups > kMaxGroups) return fail(GS_ERR_INVALID_ARGUMENT, "n_groups must lie in [0, 16]");
    if (n_groups > 0 && !groups) return fail(GS_ERR_INVALID_ARGUMENT, "groups is NULL");
    if (step < 1) return fail(GS_ERR_INVALID_ARGUMENT, "step must be >= 1");
    if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f && eps >= 0.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "bad Adam hyper-parameters");
    AdamArgs a = {};
    a.ng = n_groups;
    a.b1 = beta1;
    a.b2 = beta2;
    a.eps = eps;
    const double bc1 = 1.0 - std::pow((double)beta1, step), bc2 = 1.0 - std::pow((double)beta2, step);
    a.inv_bc2 = (float)(1.0 / bc2);
    int64_t blocks = 0;
    for (int i = 0; i < n_groups; ++i) {
        const gs_adam_group &gr = groups[i];
        if (gr.n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "group %d: n < 0", i);
        if (gr.n > 0 && (!gr.p || !gr.g || !gr.m || !gr.v))
            return fail(GS_ERR_INVALID_ARGUMENT, "group %d: NULL pointer", i);
        a.p[i] = gr.p; a.g[i] = gr.g; a.m[i] = gr.m; a.v[i] = gr.v; a.n[i] = gr.n;
        a.step[i] = (float)((double)gr.lr / bc1);
        // float4 body when the four arrays sit at the same offset from a 16-byte boundary
        // (the case for planes of [planes][N] buffers of any N)
        const uintptr_t off = reinterpret_cast<uintptr_t>(gr.p) & 15;
        const bool same = aligned(gr.p, 4) && (reinterpret_cast<uintptr_t>(gr.g) & 15) == off &&
                          (reinterpret_cast<uintptr_t>(gr.m) & 15) == off &&
                          (reinterpret_cast<uintptr_t>(gr.v) & 15) == off;
        a.head[i] = same ? (int32_t)std::min<int64_t>(((16 - off) & 15) / 4, gr.n) : 0;
        a.vec[i] = same;
        a.block0[i] = (uint32_t)blocks;
        if (gr.n > 0)
            blocks += same ? std::max<int64_t>(ceil_div((gr.n - a.head[i]) / 4, kThreads), 1) : ceil_div(gr.n, kThreads);
        if (blocks > 0x7fffffff) return fail(GS_ERR_UNSUPPORTED, "parameter groups too large");
    }
    a.block0[n_groups] = (uint32_t)blocks;
    if (blocks == 0) return GS_OK;
    k_adam<<<(unsigned)blocks, kThreads, 0, stream>>>(a);
    GS_LAUNCH_CHECK("k_adam");
    return GS_OK;
}

extern "C" gs_status gs_adam_batch_hparams(int32_t batch, double beta1, double beta2, double eps,
                                           const gs_adam_lrs *lr, gs_adam_lrs *lr_out, float *beta1_out,
                                           float *beta2_out, float *eps_out)
{
    using namespace gsi;
    if (batch < 1) return fail(GS_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (!lr || !lr_out || !beta1_out || !beta2_out || !eps_out) return fail(GS_ERR_INVALID_ARGUMENT, "NULL argument");
    const double bs = (double)batch, root = std::sqrt(bs);
    const double b1 = 1.0 - bs * (1.0 - beta1), b2 = 1.0 - bs * (1.0 - beta2);
    if (!(b1 >= 0.0 && b1 < 1.0 && b2 >= 0.0 && b2 < 1.0))
        return fail(GS_ERR_INVALID_ARGUMENT, "batch %d leaves a momentum coefficient outside [0, 1)", batch);
    const float in[6] = {lr->means, lr->log_scales, lr->quats, lr->opacity_logits, lr->sh_dc, lr->sh_rest};
    float o[6];
    for (int a = 0; a < 6; ++a) o[a] = (float)((double)in[a] * root);
    *lr_out = gs_adam_lrs{o[0], o[1], o[2], o[3], o[4], o[5]};
    *beta1_out = (float)b1;
    *beta2_out = (float)b2;
    *eps_out = (float)(eps / root);
    return GS_OK;
}
