// Error reporting and shared argument checks of the C ABI.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace {
thread_local char g_err[512] = "";
}

namespace gsi {

gs_status fail(gs_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

gs_status hip_check(hipError_t e, const char *what)
{
    if (e == hipSuccess) return GS_OK;
    return fail(GS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

gs_status check_camera(const gs_camera *cam)
{
    if (!cam) return fail(GS_ERR_INVALID_ARGUMENT, "camera is NULL");
    if (cam->width <= 0 || cam->height <= 0 || cam->width > 65536 || cam->height > 65536)
        return fail(GS_ERR_INVALID_ARGUMENT, "image size %dx%d out of range", cam->width, cam->height);
    if ((int64_t)tiles_x(cam->width) * tiles_y(cam->height) > (int64_t(1) << 24))
        return fail(GS_ERR_UNSUPPORTED, "more than 2^24 tiles");
    for (int i = 0; i < 16; ++i)
        if (!std::isfinite(cam->viewmat[i])) return fail(GS_ERR_INVALID_ARGUMENT, "viewmat not finite");
    if (!(std::isfinite(cam->fx) && std::isfinite(cam->fy) && std::isfinite(cam->cx) && std::isfinite(cam->cy)) ||
        cam->fx == 0.0f || cam->fy == 0.0f)
        return fail(GS_ERR_INVALID_ARGUMENT, "bad intrinsics");
    if (!(cam->near_z >= 0.0f) || !std::isfinite(cam->near_z))
        return fail(GS_ERR_INVALID_ARGUMENT, "near_z must be finite and >= 0");
    return GS_OK;
}

gs_status check_params(const gs_raster_params *p)
{
    if (!p) return fail(GS_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->sh_degree < 0) return fail(GS_ERR_INVALID_ARGUMENT, "sh_degree < 0");
    if (p->sh_degree > GS_MAX_SH_DEGREE) return fail(GS_ERR_UNSUPPORTED, "sh_degree %d > 3", p->sh_degree);
    if (!(p->alpha_min > 0.0f && p->alpha_min < 1.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "alpha_min must lie in (0, 1)");
    if (!(p->alpha_max >= p->alpha_min && p->alpha_max < 1.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "alpha_max must lie in [alpha_min, 1)");
    if (!(p->t_min >= 0.0f && p->t_min <= 1.0f))
        return fail(GS_ERR_INVALID_ARGUMENT, "t_min must lie in [0, 1]");
    if (std::isnan(p->depth_lo) || std::isnan(p->depth_hi))
        return fail(GS_ERR_INVALID_ARGUMENT, "depth window is NaN");
    return GS_OK;
}

}  // namespace gsi

extern "C" const char *gs_last_error(void) { return g_err; }
