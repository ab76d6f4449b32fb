/*
 * gs_oracle.c -- plain, slow, single-threaded CPU reference for the 3D Gaussian
 * splatting training step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library; both sides are written independently from the same
 * definitions and compared in the tests.
 *
 * Precision: double throughout, except where the method itself stores or
 * decides in single precision:
 *   - the projected 2D record (pixel mean, conic, opacity, colour) is a record
 *     of 4-byte scalars ("Scaling 3D Gaussian Splatting with Distributed
 *     Compute", step 5 of the walkthrough: about twelve 4-byte scalars per
 *     (camera, Gaussian) pair).  The oracle projects in double and rounds the
 *     record to float; compositing then runs in double on those values.
 *   - the depth sort key is the float32 camera-space depth produced by an
 *     explicitly rounded expression (see depth_key()), so that the per-tile
 *     order is an integer decision both implementations take identically.
 *   - tile rectangles are computed with float32 operations (rect_f32()), the
 *     same precision as the binning kernel.
 *
 * Sources (page titles; sections / equations):
 *   [Splaxel]   "Splaxel: Efficient Distributed Training of 3D Gaussian
 *               Splatting for Large-scale Scene Reconstruction via Pixel-level
 *               Communication", section 2 (Background: Sigma = R S S^T R^T,
 *               frustum culling by the mean, Sigma2D = J W Sigma W^T J^T,
 *               depth sort), section 4.2 (convex partitions preserve the
 *               global blending order), section 4.3 (saturation redundancy,
 *               epsilon = 1e-4).
 *   [ByteSplat] "ByteSplat: Efficient Distributed 3D Gaussian Splatting
 *               Training via Intra- and Inter-GPU communication reduction",
 *               section 2.1 (Eq. 1 front-to-back compositing with
 *               alpha-checking and termination at theta_T; Eq. 3 per
 *               pixel-Gaussian partial gradient; Eq. 4 aggregation; backward
 *               through projection and colour), section 3 Insight 4 and
 *               section 6 (zero-gradient elision: all fields exactly zero).
 *   [gsplat]    "Scaling 3D Gaussian Splatting with Distributed Compute"
 *               (ROCm blog): parameterisation (mean, scale + quaternion, SH
 *               colour, opacity), SH evaluated to RGB per camera, L1 term of
 *               the loss, Adam with eps 1e-15 and betas (0.9, 0.999) at
 *               batch size 1.
 *
 * Readings where the pages are silent are listed in the design notes; the
 * ones this file implements are marked "reading:" at the point of use.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_TILE 16
#define ORC_RADIUS_CAP (1 << 20)
#define ORC_MAX_DEG 4

/* ------------------------------------------------------------------ camera */

typedef struct {
    double R[3][3];   /* world -> camera rotation (rows of the view matrix) */
    double t[3];
    double fx, fy, cx, cy;
    int W, H;
    double near_z;
    float r2[3], t2;  /* float row 2 of the view matrix (depth key) */
    double campos[3]; /* camera centre in world coordinates, -R^T t */
} ocam;

static void cam_init(ocam *c, const double *viewmat, const double *intr, int W, int H, double near_z)
{
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j) c->R[i][j] = (double)viewmat[4 * i + j];
        c->t[i] = (double)viewmat[4 * i + 3];
    }
    c->fx = intr[0]; c->fy = intr[1]; c->cx = intr[2]; c->cy = intr[3];
    c->W = W; c->H = H; c->near_z = near_z;
    c->r2[0] = (float)viewmat[8]; c->r2[1] = (float)viewmat[9]; c->r2[2] = (float)viewmat[10];
    c->t2 = (float)viewmat[11];
    for (int j = 0; j < 3; ++j)
        c->campos[j] = -(c->R[0][j] * c->t[0] + c->R[1][j] * c->t[1] + c->R[2][j] * c->t[2]);
}

/* Camera-space depth as a float32 value: ((r20*x) fused-multiply-added with
 * r21*y, then with r22*z), plus t2, every step rounded to nearest float.  Its
 * bit pattern (a positive float) orders like an unsigned integer and is the
 * depth part of the sort key.  Built with -ffp-contract=off so that the
 * product and the final sum are separately rounded. */
static float depth_key(const ocam *c, float x, float y, float z)
{
    float p = c->r2[0] * x;
    float s = fmaf(c->r2[1], y, p);
    s = fmaf(c->r2[2], z, s);
    return s + c->t2;
}

/* ---------------------------------------------------- real SH basis (any l) */

/* Coefficients (ascending powers) of the Legendre polynomial P_l, from
 * Bonnet's recursion (l+1) P_{l+1} = (2l+1) z P_l - l P_{l-1}. */
static void legendre_coeffs(int l, double *out)
{
    double a[ORC_MAX_DEG + 2] = {0}, b[ORC_MAX_DEG + 2] = {0}, c[ORC_MAX_DEG + 2];
    a[0] = 1.0;                 /* P_0 */
    b[1] = 1.0;                 /* P_1 */
    if (l == 0) { memcpy(out, a, sizeof(double) * (l + 1)); return; }
    for (int k = 1; k < l; ++k) {
        memset(c, 0, sizeof(c));
        for (int i = 0; i <= k; ++i) c[i + 1] += (2.0 * k + 1.0) * b[i];
        for (int i = 0; i <= k - 1; ++i) c[i] -= (double)k * a[i];
        for (int i = 0; i <= k + 1; ++i) c[i] /= (double)(k + 1);
        memcpy(a, b, sizeof(a));
        memcpy(b, c, sizeof(b));
    }
    memcpy(out, b, sizeof(double) * (l + 1));
}

/* m-th derivative of the polynomial with coefficients c[0..deg] at z. */
static double poly_deriv(const double *c, int deg, int m, double z)
{
    double s = 0.0, zp = 1.0;
    for (int k = m; k <= deg; ++k) {
        double f = 1.0;
        for (int j = 0; j < m; ++j) f *= (double)(k - j);
        s += c[k] * f * zp;
        zp *= z;
    }
    return s;
}

static double factorial(int n)
{
    double f = 1.0;
    for (int i = 2; i <= n; ++i) f *= i;
    return f;
}

/* Real orthonormal spherical harmonics at the unit vector d = (x, y, z),
 * index l*l + l + m, without the Condon-Shortley phase:
 *   Y_lm = sqrt(2) K_lm cos(m phi) P_l^m(cos theta)    m > 0
 *   Y_lm = sqrt(2) K_lm sin(|m| phi) P_l^|m|(cos theta) m < 0
 *   Y_l0 = K_l0 P_l(cos theta)
 *   K_lm = sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!)
 * Written in Cartesian form: P_l^m(z) = (1-z^2)^(m/2) d^m P_l/dz^m and
 * sin^m(theta) e^(i m phi) = (x + i y)^m, so
 *   Y_lm = N_lm * (d^|m| P_l/dz^|m|)(z) * {Re, 1, Im}((x + i y)^|m|).
 * If grad != NULL, grad[3*k + j] receives dY_k/d(x, y, z)_j of that polynomial
 * (its tangential part is the derivative on the sphere).
 * reading: real orthonormal basis, no Condon-Shortley phase. */
static void sh_basis(int deg, const double d[3], double *Y, double *grad)
{
    const double x = d[0], y = d[1], z = d[2];
    /* powers of w = x + i y */
    double wr[ORC_MAX_DEG + 1], wi[ORC_MAX_DEG + 1];
    wr[0] = 1.0; wi[0] = 0.0;
    for (int m = 1; m <= deg; ++m) {
        wr[m] = wr[m - 1] * x - wi[m - 1] * y;
        wi[m] = wr[m - 1] * y + wi[m - 1] * x;
    }
    for (int l = 0; l <= deg; ++l) {
        double pc[ORC_MAX_DEG + 1];
        legendre_coeffs(l, pc);
        for (int m = -l; m <= l; ++m) {
            const int am = m < 0 ? -m : m;
            double N = sqrt((2.0 * l + 1.0) / (4.0 * M_PI) * factorial(l - am) / factorial(l + am));
            if (m != 0) N *= sqrt(2.0);
            const double Q = poly_deriv(pc, l, am, z);
            const double Qz = poly_deriv(pc, l, am + 1, z);
            double Wv, Wx, Wy;
            if (m > 0) {
                Wv = wr[am];
                Wx = am * wr[am - 1];
                Wy = -am * wi[am - 1];
            } else if (m < 0) {
                Wv = wi[am];
                Wx = am * wi[am - 1];
                Wy = am * wr[am - 1];
            } else {
                Wv = 1.0; Wx = 0.0; Wy = 0.0;
            }
            const int k = l * l + l + m;
            Y[k] = N * Q * Wv;
            if (grad) {
                grad[3 * k + 0] = N * Q * Wx;
                grad[3 * k + 1] = N * Q * Wy;
                grad[3 * k + 2] = N * Qz * Wv;
            }
        }
    }
}

/* exported for the basis pins (orthonormality, addition theorem) */
void orc_sh_basis(int deg, const double *dir, double *Y, double *grad)
{
    sh_basis(deg, dir, Y, grad);
}

/* ------------------------------------------------------------ projection */

/* Rotation matrix of the unit quaternion (w, x, y, z) (Hamilton convention).
 * reading: quaternion stored as (w, x, y, z) and normalised in the forward. */
static void quat_to_rot(const double q[4], double R[3][3])
{
    const double w = q[0], x = q[1], y = q[2], z = q[3];
    R[0][0] = 1 - 2 * (y * y + z * z); R[0][1] = 2 * (x * y - w * z);     R[0][2] = 2 * (x * z + w * y);
    R[1][0] = 2 * (x * y + w * z);     R[1][1] = 1 - 2 * (x * x + z * z); R[1][2] = 2 * (y * z - w * x);
    R[2][0] = 2 * (x * z - w * y);     R[2][1] = 2 * (y * z + w * x);     R[2][2] = 1 - 2 * (x * x + y * y);
}

/* exported for the rotation pin */
void orc_quat_to_rot(const double *q, double *R9)
{
    double R[3][3];
    quat_to_rot(q, R);
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) R9[3 * i + j] = R[i][j];
}

typedef struct {
    int vis;            /* survived culling */
    int marginal;       /* a culling decision sits within rounding distance of its threshold */
    double mu[3], s[3], qn[4], qnorm, o;
    double Rq[3][3], M[3][3], Sig[3][3];
    double X, Y, Z;
    double u, v;
    double J[2][3], T[2][3];
    double a, b, c, det;
    double A, B, C;
    double dir[3], dist, Ysh[(ORC_MAX_DEG + 1) * (ORC_MAX_DEG + 1)];
    double color[3];
    float dkey;
    int32_t rx, ry;
} oproj;

static int all_finite(const double *x, int n)
{
    for (int i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* Sigmoid of the opacity logit, rounded to the float record value if asked.
 * reading: opacities are stored as logits and activated with the logistic function. */
static double opacity_of(double logit, int round_record)
{
    const double o = 1.0 / (1.0 + exp(-logit));
    return round_record ? (double)(float)o : o;
}

/*
 * Project Gaussian i.  Implements, in order:
 *   activations  s = exp(log_s), o = sigmoid(logit), q^ = q/|q|;
 *   Sigma = M M^T with M = R(q^) diag(s)            [Splaxel sec. 2];
 *   p = W mu + t (world -> camera);
 *   frustum culling by the mean: z > near_z and the projected mean inside
 *     [0, W) x [0, H)                                [Splaxel sec. 2, "Projection"];
 *   Sigma2D = J W Sigma W^T J^T, J the Jacobian of the pinhole map at p
 *                                                    [Splaxel sec. 2];
 *   conic = Sigma2D^{-1}; cull if det <= 0 or o < alpha_min;
 *   radii: the alpha >= alpha_min ellipse {d : d^T conic d <= 2 ln(o/alpha_min)}
 *     has half-extents sqrt(2 ln(o/alpha_min) Sigma2D_xx) (and _yy); radius =
 *     ceil of that, at least 1, capped (reading);
 *   colour = sum_lm k_lm Y_lm(v^), v^ = unit vector from the camera centre to
 *     the mean, no offset and no clamp (reading) [gsplat blog, SH colour].
 */
static void project_one(const ocam *cam, int deg, int64_t n, int64_t i,
                        const double *means, const double *log_scales, const double *quats,
                        const double *logits, const double *sh, double alpha_min,
                        float depth_lo, float depth_hi, int round_record, oproj *P)
{
    const int K = (deg + 1) * (deg + 1);
    memset(P, 0, sizeof(*P));
    double raw[3 + 3 + 4 + 1];
    for (int j = 0; j < 3; ++j) raw[j] = means[j * n + i];
    for (int j = 0; j < 3; ++j) raw[3 + j] = log_scales[j * n + i];
    for (int j = 0; j < 4; ++j) raw[6 + j] = quats[j * n + i];
    raw[10] = logits[i];
    int finite = all_finite(raw, 11);
    for (int k = 0; k < 3 * K && finite; ++k) finite = isfinite(sh[(int64_t)k * n + i]);
    if (!finite) return;

    for (int j = 0; j < 3; ++j) { P->mu[j] = raw[j]; P->s[j] = exp(raw[3 + j]); }
    P->qnorm = sqrt(raw[6] * raw[6] + raw[7] * raw[7] + raw[8] * raw[8] + raw[9] * raw[9]);
    if (!(P->qnorm > 0.0)) return;
    for (int j = 0; j < 4; ++j) P->qn[j] = raw[6 + j] / P->qnorm;
    P->o = opacity_of(raw[10], round_record);

    /* depth window of a partial render; the key is the float expression */
    P->dkey = depth_key(cam, (float)means[0 * n + i], (float)means[1 * n + i], (float)means[2 * n + i]);
    if (!(P->dkey >= depth_lo && P->dkey < depth_hi)) return;

    P->X = cam->R[0][0] * P->mu[0] + cam->R[0][1] * P->mu[1] + cam->R[0][2] * P->mu[2] + cam->t[0];
    P->Y = cam->R[1][0] * P->mu[0] + cam->R[1][1] * P->mu[1] + cam->R[1][2] * P->mu[2] + cam->t[1];
    P->Z = cam->R[2][0] * P->mu[0] + cam->R[2][1] * P->mu[1] + cam->R[2][2] * P->mu[2] + cam->t[2];
    if (fabs(P->Z - cam->near_z) <= 1e-9 * fabs(cam->near_z)) P->marginal = 1;
    if (!(P->Z > cam->near_z)) return;
    P->u = cam->fx * P->X / P->Z + cam->cx;
    P->v = cam->fy * P->Y / P->Z + cam->cy;
    {
        const double eps = 1e-7;
        if (fabs(P->u) < eps || fabs(P->u - cam->W) < eps || fabs(P->v) < eps || fabs(P->v - cam->H) < eps)
            P->marginal = 1;
    }
    /* reading: culling uses the projected mean only, no guard band */
    if (!(P->u >= 0.0 && P->u < cam->W && P->v >= 0.0 && P->v < cam->H)) return;

    quat_to_rot(P->qn, P->Rq);
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) P->M[r][c] = P->Rq[r][c] * P->s[c];
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k) acc += P->M[r][k] * P->M[c][k];
            P->Sig[r][c] = acc;
        }
    const double Z = P->Z;
    P->J[0][0] = cam->fx / Z; P->J[0][1] = 0.0;          P->J[0][2] = -cam->fx * P->X / (Z * Z);
    P->J[1][0] = 0.0;         P->J[1][1] = cam->fy / Z;  P->J[1][2] = -cam->fy * P->Y / (Z * Z);
    for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 3; ++c) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k) acc += P->J[r][k] * cam->R[k][c];
            P->T[r][c] = acc;
        }
    double TS[2][3];
    for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 3; ++c) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k) acc += P->T[r][k] * P->Sig[k][c];
            TS[r][c] = acc;
        }
    double S2[2][2];
    for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 2; ++c) {
            double acc = 0.0;
            for (int k = 0; k < 3; ++k) acc += TS[r][k] * P->T[c][k];
            S2[r][c] = acc;
        }
    P->a = S2[0][0]; P->b = 0.5 * (S2[0][1] + S2[1][0]); P->c = S2[1][1];
    P->det = P->a * P->c - P->b * P->b;
    if (fabs(P->det) <= 1e-9 * fabs(P->a * P->c)) P->marginal = 1;
    if (!(P->det > 0.0)) return;
    P->A = P->c / P->det; P->B = -P->b / P->det; P->C = P->a / P->det;

    if (fabs(P->o - alpha_min) <= 4.0 * (double)FLT_EPSILON * alpha_min) P->marginal = 1;
    if (!(P->o >= alpha_min)) return;

    const double lnr = 2.0 * log(P->o / alpha_min);
    double ex = ceil(sqrt(lnr * P->a)), ey = ceil(sqrt(lnr * P->c));
    if (ex < 1.0) ex = 1.0;
    if (ey < 1.0) ey = 1.0;
    if (ex > ORC_RADIUS_CAP) ex = ORC_RADIUS_CAP;
    if (ey > ORC_RADIUS_CAP) ey = ORC_RADIUS_CAP;
    P->rx = (int32_t)ex; P->ry = (int32_t)ey;

    for (int j = 0; j < 3; ++j) P->dir[j] = P->mu[j] - cam->campos[j];
    P->dist = sqrt(P->dir[0] * P->dir[0] + P->dir[1] * P->dir[1] + P->dir[2] * P->dir[2]);
    double vhat[3] = {P->dir[0] / P->dist, P->dir[1] / P->dist, P->dir[2] / P->dist};
    sh_basis(deg, vhat, P->Ysh, NULL);
    for (int ch = 0; ch < 3; ++ch) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += sh[(int64_t)(k * 3 + ch) * n + i] * P->Ysh[k];
        P->color[ch] = acc;
    }
    P->vis = 1;
}

/*
 * Forward projection of all Gaussians.
 * Outputs per Gaussian: vis, rec[n][9] = (u, v, A, B, C, o, r, g, b) -- each
 * value rounded to float when round_record != 0 (the method's 4-byte record),
 * exact doubles otherwise (for finite-difference checks) --, depth key
 * (float), radii [n][2] (0,0 if culled) and the marginal flag.
 */
int orc_project(int64_t n, int deg,
                const double *means, const double *log_scales, const double *quats,
                const double *logits, const double *sh,
                const double *viewmat, const double *intr, int W, int H, double near_z,
                float alpha_min, float depth_lo, float depth_hi, int round_record,
                int32_t *vis, double *rec, float *dkey, int32_t *radii, uint8_t *marginal)
{
    if (deg < 0 || deg > ORC_MAX_DEG) return -1;
    ocam cam;
    cam_init(&cam, viewmat, intr, W, H, near_z);
    oproj P;
    for (int64_t i = 0; i < n; ++i) {
        project_one(&cam, deg, n, i, means, log_scales, quats, logits, sh, (double)alpha_min,
                    depth_lo, depth_hi, round_record, &P);
        vis[i] = P.vis;
        marginal[i] = (uint8_t)P.marginal;
        dkey[i] = P.dkey;
        double *r = rec + 9 * i;
        if (P.vis) {
            r[0] = P.u; r[1] = P.v; r[2] = P.A; r[3] = P.B; r[4] = P.C; r[5] = P.o;
            r[6] = P.color[0]; r[7] = P.color[1]; r[8] = P.color[2];
            if (round_record)
                for (int k = 0; k < 9; ++k) r[k] = (double)(float)r[k];
            radii[2 * i] = P.rx; radii[2 * i + 1] = P.ry;
        } else {
            for (int k = 0; k < 9; ++k) r[k] = 0.0;
            radii[2 * i] = 0; radii[2 * i + 1] = 0;
        }
    }
    return 0;
}

/* -------------------------------------------------------------- binning */

/* Tile rectangle [x0,x1) x [y0,y1) of a Gaussian with float pixel mean (u, v)
 * and integer radii: every 16x16 tile that the box [u-rx, u+rx] x [v-ry, v+ry]
 * touches, clamped to the tile grid.  All arithmetic in float32 (the binning
 * decision is taken in the kernel's precision); division by 16 is exact. */
static void rect_f32(float u, float v, int32_t rx, int32_t ry, int TX, int TY,
                     int *x0, int *x1, int *y0, int *y1)
{
    float fx0 = floorf((u - (float)rx) / 16.0f);
    float fx1 = floorf((u + (float)rx) / 16.0f) + 1.0f;
    float fy0 = floorf((v - (float)ry) / 16.0f);
    float fy1 = floorf((v + (float)ry) / 16.0f) + 1.0f;
    fx0 = fminf(fmaxf(fx0, 0.0f), (float)TX);
    fx1 = fminf(fmaxf(fx1, 0.0f), (float)TX);
    fy0 = fminf(fmaxf(fy0, 0.0f), (float)TY);
    fy1 = fminf(fmaxf(fy1, 0.0f), (float)TY);
    *x0 = (int)fx0; *x1 = (int)fx1; *y0 = (int)fy0; *y1 = (int)fy1;
}

typedef struct { uint64_t key; uint32_t id; } kv;

static int cmp_kv(const void *pa, const void *pb)
{
    const kv *a = (const kv *)pa, *b = (const kv *)pb;
    if (a->key != b->key) return a->key < b->key ? -1 : 1;
    return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);
}

static uint32_t fbits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/*
 * Tile binning from float projected inputs [ByteSplat sec. 2.1 "Projection",
 * "Sorting"]: every visible Gaussian (both radii > 0) emits one entry per
 * tile of its rectangle, key = tile id << 32 | depth bits, tile id row-major;
 * entries sorted by (key, Gaussian index) with the library sort; per-tile
 * [start, end) ranges.  Returns K (the number of entries); if K > cap only
 * tiles_touched and the return value are written.
 */
int64_t orc_bin_f32(int64_t n, const float *means2d, const int32_t *radii, const float *depth,
                    int W, int H, int32_t *tiles_touched, int64_t cap,
                    uint64_t *keys, uint32_t *ids, int32_t *ranges)
{
    const int TX = (W + ORC_TILE - 1) / ORC_TILE, TY = (H + ORC_TILE - 1) / ORC_TILE;
    int64_t K = 0;
    for (int64_t i = 0; i < n; ++i) {
        int cnt = 0;
        if (radii[2 * i] > 0 && radii[2 * i + 1] > 0) {
            int x0, x1, y0, y1;
            rect_f32(means2d[2 * i], means2d[2 * i + 1], radii[2 * i], radii[2 * i + 1], TX, TY,
                     &x0, &x1, &y0, &y1);
            cnt = (x1 - x0) * (y1 - y0);
        }
        tiles_touched[i] = cnt;
        K += cnt;
    }
    if (K > cap) return K;
    kv *e = (kv *)malloc(sizeof(kv) * (K > 0 ? K : 1));
    int64_t p = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (tiles_touched[i] == 0) continue;
        int x0, x1, y0, y1;
        rect_f32(means2d[2 * i], means2d[2 * i + 1], radii[2 * i], radii[2 * i + 1], TX, TY,
                 &x0, &x1, &y0, &y1);
        for (int ty = y0; ty < y1; ++ty)
            for (int tx = x0; tx < x1; ++tx) {
                e[p].key = ((uint64_t)(ty * TX + tx) << 32) | fbits(depth[i]);
                e[p].id = (uint32_t)i;
                ++p;
            }
    }
    qsort(e, (size_t)K, sizeof(kv), cmp_kv);
    const int T = TX * TY;
    int64_t k = 0;
    for (int t = 0; t <= T; ++t) {
        while (k < K && (int64_t)(e[k].key >> 32) < t) ++k;
        ranges[t] = (int32_t)k;
    }
    for (int64_t j = 0; j < K; ++j) { keys[j] = e[j].key; ids[j] = e[j].id; }
    free(e);
    return K;
}

/* ----------------------------------------------------------- compositing */

typedef struct {
    int T;                 /* number of lists */
    int64_t *start;        /* [T+1] */
    uint32_t *ids;         /* Gaussian indices, each list sorted by (depth key bits, index) */
} olists;

/* Visible Gaussians sorted by (depth key bits, index): Splaxel sec. 2
 * "Sorting" / ByteSplat sec. 2.1 "Sorting"; reading: ties broken by index. */
static uint32_t *sorted_visible(int64_t n, const int32_t *vis, const float *dkey, int64_t *nv)
{
    kv *e = (kv *)malloc(sizeof(kv) * (n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i)
        if (vis[i]) { e[m].key = fbits(dkey[i]); e[m].id = (uint32_t)i; ++m; }
    qsort(e, (size_t)m, sizeof(kv), cmp_kv);
    uint32_t *out = (uint32_t *)malloc(sizeof(uint32_t) * (m > 0 ? m : 1));
    for (int64_t j = 0; j < m; ++j) out[j] = e[j].id;
    free(e);
    *nv = m;
    return out;
}

/* Candidate lists.  literal != 0: one list holding every visible Gaussian
 * (the plain per-pixel definition).  Otherwise one list per 16x16 tile with
 * the Gaussians whose tile rectangle covers it.  A Gaussian outside a pixel's
 * alpha >= alpha_min ellipse contributes exactly nothing there, so both give
 * the same image; the tile form is what the method traverses. */
static void build_lists(int64_t n, const int32_t *vis, const double *rec, const float *dkey,
                        const int32_t *radii, int W, int H, int literal, olists *L)
{
    int64_t nv;
    uint32_t *order = sorted_visible(n, vis, dkey, &nv);
    if (literal) {
        L->T = 1;
        L->start = (int64_t *)malloc(sizeof(int64_t) * 2);
        L->start[0] = 0; L->start[1] = nv;
        L->ids = order;
        return;
    }
    const int TX = (W + ORC_TILE - 1) / ORC_TILE, TY = (H + ORC_TILE - 1) / ORC_TILE;
    L->T = TX * TY;
    int64_t *cnt = (int64_t *)calloc((size_t)L->T + 1, sizeof(int64_t));
    for (int64_t j = 0; j < nv; ++j) {
        const uint32_t i = order[j];
        int x0, x1, y0, y1;
        rect_f32((float)rec[9 * i], (float)rec[9 * i + 1], radii[2 * i], radii[2 * i + 1], TX, TY, &x0, &x1, &y0, &y1);
        for (int ty = y0; ty < y1; ++ty)
            for (int tx = x0; tx < x1; ++tx) cnt[ty * TX + tx + 1]++;
    }
    for (int t = 0; t < L->T; ++t) cnt[t + 1] += cnt[t];
    L->start = cnt;
    L->ids = (uint32_t *)malloc(sizeof(uint32_t) * (cnt[L->T] > 0 ? cnt[L->T] : 1));
    int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * L->T);
    memcpy(fill, cnt, sizeof(int64_t) * L->T);
    for (int64_t j = 0; j < nv; ++j) {
        const uint32_t i = order[j];
        int x0, x1, y0, y1;
        rect_f32((float)rec[9 * i], (float)rec[9 * i + 1], radii[2 * i], radii[2 * i + 1], TX, TY, &x0, &x1, &y0, &y1);
        for (int ty = y0; ty < y1; ++ty)
            for (int tx = x0; tx < x1; ++tx) L->ids[fill[ty * TX + tx]++] = i;
    }
    free(fill);
    free(order);
}

static void free_lists(olists *L)
{
    free(L->start);
    free(L->ids);
}

typedef struct {
    uint32_t id;
    double T, alpha, ge, raw, dx, dy;
} ohit;

/* Tie thresholds: a pixel is a "tie" if one of its decisions is closer to its
 * threshold than the float32 evaluation error of the GPU path can resolve. */
#define TIE_ALPHA_REL 1e-5
#define TIE_ALPHA_MIN_T 1e-3
#define TIE_T_REL 1e-3

/*
 * One pixel, front to back [ByteSplat Eq. 1]:
 *   T_1 = 1; for each list entry i in order:
 *     stop if T_i < theta_T                       (termination, reading: checked
 *                                                  before each entry)
 *     alpha_i = min(alpha_max, o_i exp(power_i)),
 *     power_i = -1/2 (A dx^2 + C dy^2) - B dx dy, (dx, dy) = pixel centre - mean
 *                                                 (reading: pixel centres at +0.5)
 *     skip if alpha_i < alpha_min                 (the alpha-check)
 *     C += T_i alpha_i c_i;  T_{i+1} = T_i (1 - alpha_i)
 * N_p = number of list entries traversed.  Accepted entries are appended to
 * hits (for the backward) if hits != NULL.
 */
static void shade_pixel(const olists *L, int list, const double *rec, double px, double py,
                        double amin, double amax, double tmin, double out_c[3], double *out_t,
                        int32_t *out_n, int *tie, ohit *hits, int64_t *nhits)
{
    double T = 1.0, Cc[3] = {0, 0, 0};
    int64_t n = 0, nh = 0;
    const int64_t b = L->start[list], e = L->start[list + 1];
    int t = 0;
    for (int64_t k = b; k < e; ++k) {
        if (tmin > 0.0 && fabs(T / tmin - 1.0) < TIE_T_REL) t = 1;
        if (T < tmin) break;
        ++n;
        const uint32_t i = L->ids[k];
        const double *r = rec + 9 * (int64_t)i;
        const double dx = px - r[0], dy = py - r[1];
        const double A = r[2], B = r[3], C = r[4], o = r[5];
        const double power = -0.5 * (A * dx * dx + C * dy * dy) - B * dx * dy;
        const double ge = exp(power);
        const double raw = o * ge;
        if (fabs(raw / amin - 1.0) < TIE_ALPHA_REL && T >= TIE_ALPHA_MIN_T) t = 1;
        const double alpha = raw < amax ? raw : amax;
        if (alpha < amin) continue;
        for (int ch = 0; ch < 3; ++ch) Cc[ch] += T * alpha * r[6 + ch];
        if (hits) {
            ohit *h = &hits[nh];
            h->id = i; h->T = T; h->alpha = alpha; h->ge = ge; h->raw = raw; h->dx = dx; h->dy = dy;
        }
        ++nh;
        T *= (1.0 - alpha);
    }
    if (tmin > 0.0 && fabs(T / tmin - 1.0) < TIE_T_REL) t = 1;
    for (int ch = 0; ch < 3; ++ch) out_c[ch] = Cc[ch];
    *out_t = T;
    *out_n = (int32_t)n;
    *tie = t;
    if (nhits) *nhits = nh;
}

static int list_of_pixel(int literal, int W, int x, int y)
{
    if (literal) return 0;
    const int TX = (W + ORC_TILE - 1) / ORC_TILE;
    return (y / ORC_TILE) * TX + (x / ORC_TILE);
}

/*
 * Render the given pixels (pix = [npix][2] of (x, y)).  Outputs per listed
 * pixel: color [npix][3], t_final [npix], n_trav [npix], tie [npix].
 * Gaussians flagged marginal by the projection also mark as tie every pixel of
 * their box.  rec/dkey/radii/vis/marginal come from orc_project.
 */
int orc_render(int64_t n, const int32_t *vis, const double *rec, const float *dkey,
               const int32_t *radii, const uint8_t *marginal, int W, int H,
               float alpha_min, float alpha_max, float t_min, int literal,
               int64_t npix, const int32_t *pix,
               double *color, double *t_final, int32_t *n_trav, uint8_t *tie)
{
    olists L;
    build_lists(n, vis, rec, dkey, radii, W, H, literal, &L);
    for (int64_t p = 0; p < npix; ++p) {
        const int x = pix[2 * p], y = pix[2 * p + 1];
        int t;
        shade_pixel(&L, list_of_pixel(literal, W, x, y), rec, x + 0.5, y + 0.5,
                    (double)alpha_min, (double)alpha_max, (double)t_min,
                    color + 3 * p, t_final + p, n_trav + p, &t, NULL, NULL);
        tie[p] = (uint8_t)t;
    }
    free_lists(&L);
    /* marginal culling decisions: mark their box (they may be culled here but
     * not elsewhere, so use a generous box around the rounded mean) */
    for (int64_t i = 0; i < n; ++i) {
        if (!marginal[i]) continue;
        for (int64_t p = 0; p < npix; ++p) {
            const double dx = pix[2 * p] + 0.5 - rec[9 * i];
            const double dy = pix[2 * p + 1] + 0.5 - rec[9 * i + 1];
            const double rx = radii[2 * i] > 0 ? radii[2 * i] + 1.0 : 64.0;
            const double ry = radii[2 * i + 1] > 0 ? radii[2 * i + 1] + 1.0 : 64.0;
            if (fabs(dx) <= rx && fabs(dy) <= ry) tie[p] = 1;
        }
    }
    return 0;
}

/* Gradient field order of the screen-space record (grads2d rows). */
enum { G_U = 0, G_V, G_A, G_B, G_C, G_O, G_R, G_G, G_BL, G_N };

/*
 * Backward through compositing [ByteSplat Eq. 3 and Eq. 4].  For every listed
 * pixel, with G = dL/dC(p) and G_T = dL/dT_final(p) (nullable), walk the
 * accepted entries back to front:
 *   dL/dc_i     += T_i alpha_i G
 *   dL/dalpha_i  = T_i (c_i - B_i) . G - G_T T_final / (1 - alpha_i),
 *                  B_i the normalised colour behind i: B = 0 after the last
 *                  entry, B_{i-1} = alpha_i c_i + (1 - alpha_i) B_i
 *   unclamped alpha (o e^power < alpha_max): dL/do += dL/dalpha e^power,
 *                  dL/dpower = dL/dalpha alpha; clamped: both 0 (reading)
 *   dA += -dx^2/2 dpower, dB += -dx dy dpower, dC += -dy^2/2 dpower,
 *   du += (A dx + B dy) dpower, dv += (B dx + C dy) dpower.
 * grads2d [9][n] (double) is accumulated (sum over pixels, Eq. 4).
 */
int orc_raster_backward(int64_t n, const int32_t *vis, const double *rec, const float *dkey,
                        const int32_t *radii, int W, int H,
                        float alpha_min, float alpha_max, float t_min,
                        int64_t npix, const int32_t *pix, const double *G, const double *GT,
                        double *grads2d)
{
    olists L;
    build_lists(n, vis, rec, dkey, radii, W, H, 0, &L);
    int64_t maxlen = 0;
    for (int t = 0; t < L.T; ++t)
        if (L.start[t + 1] - L.start[t] > maxlen) maxlen = L.start[t + 1] - L.start[t];
    ohit *hits = (ohit *)malloc(sizeof(ohit) * (maxlen > 0 ? maxlen : 1));
    const double amin = alpha_min, amax = alpha_max;
    for (int64_t p = 0; p < npix; ++p) {
        const int x = pix[2 * p], y = pix[2 * p + 1];
        double col[3], Tf;
        int32_t nt;
        int tie;
        int64_t nh;
        shade_pixel(&L, list_of_pixel(0, W, x, y), rec, x + 0.5, y + 0.5, amin, amax,
                    (double)t_min, col, &Tf, &nt, &tie, hits, &nh);
        const double g0 = G[3 * p], g1 = G[3 * p + 1], g2 = G[3 * p + 2];
        const double gt = GT ? GT[p] : 0.0;
        double Bc[3] = {0, 0, 0};
        for (int64_t h = nh - 1; h >= 0; --h) {
            const ohit *H_ = &hits[h];
            const double *r = rec + 9 * (int64_t)H_->id;
            const double c[3] = {r[6], r[7], r[8]};
            const double A = r[2], B = r[3], C = r[4];
            const double Ti = H_->T, al = H_->alpha;
            double *gr = grads2d;
            const int64_t id = H_->id;
            gr[G_R * n + id] += Ti * al * g0;
            gr[G_G * n + id] += Ti * al * g1;
            gr[G_BL * n + id] += Ti * al * g2;
            double dal = Ti * ((c[0] - Bc[0]) * g0 + (c[1] - Bc[1]) * g1 + (c[2] - Bc[2]) * g2);
            dal -= gt * Tf / (1.0 - al);
            if (H_->raw < amax) {
                const double dpow = dal * al;
                gr[G_O * n + id] += dal * H_->ge;
                const double dx = H_->dx, dy = H_->dy;
                gr[G_A * n + id] += -0.5 * dx * dx * dpow;
                gr[G_B * n + id] += -dx * dy * dpow;
                gr[G_C * n + id] += -0.5 * dy * dy * dpow;
                gr[G_U * n + id] += (A * dx + B * dy) * dpow;
                gr[G_V * n + id] += (B * dx + C * dy) * dpow;
            }
            for (int ch = 0; ch < 3; ++ch) Bc[ch] = al * c[ch] + (1.0 - al) * Bc[ch];
        }
    }
    free(hits);
    free_lists(&L);
    return 0;
}

/*
 * Backward through projection and colour evaluation [ByteSplat sec. 2.1,
 * "Gradient Aggregation and Update": the aggregated screen-space gradients are
 * backpropagated through projection and colour evaluation].  Exact chain rule
 * of project_one (the float rounding of the record is treated as identity):
 *   conic:   G_Q = [[dA, dB/2], [dB/2, dC]], G_S2 = -Q G_Q Q
 *   EWA:     Sigma2D = T Sigma T^T, T = J W:  G_T = 2 G_S2 T Sigma,
 *            G_Sigma = T^T G_S2 T;  G_J = G_T W^T
 *   pinhole: J and (u, v) depend on p = (X, Y, Z); dmu = W^T dp
 *   Sigma = M M^T: G_M = 2 G_Sigma M; M = R diag(s): ds_k = sum_i G_M[i][k] R[i][k],
 *            dlog_s = s * ds; G_R = G_M diag(s) -> dq^ -> dq = (dq^ - q^(q^.dq^))/|q|
 *   opacity: dlogit = do * o (1 - o)
 *   colour:  dk_lm = Y_lm(v^) dc; dv^ = sum_lm k_lm . dc grad Y_lm,
 *            dmu += (I - v^ v^T) dv^ / |mu - campos|
 * Culled Gaussians get zero gradients.  Outputs overwrite (double planes).
 */
int orc_project_backward(int64_t n, int deg,
                         const double *means, const double *log_scales, const double *quats,
                         const double *logits, const double *sh,
                         const double *viewmat, const double *intr, int W, int H, double near_z,
                         float alpha_min, float depth_lo, float depth_hi, int round_record,
                         const double *grads2d,
                         double *d_means, double *d_log_scales, double *d_quats,
                         double *d_logits, double *d_sh)
{
    if (deg < 0 || deg > ORC_MAX_DEG) return -1;
    const int K = (deg + 1) * (deg + 1);
    ocam cam;
    cam_init(&cam, viewmat, intr, W, H, near_z);
    oproj P;
    for (int64_t i = 0; i < n; ++i) {
        project_one(&cam, deg, n, i, means, log_scales, quats, logits, sh, (double)alpha_min,
                    depth_lo, depth_hi, round_record, &P);
        for (int j = 0; j < 3; ++j) { d_means[j * n + i] = 0.0; d_log_scales[j * n + i] = 0.0; }
        for (int j = 0; j < 4; ++j) d_quats[j * n + i] = 0.0;
        d_logits[i] = 0.0;
        for (int k = 0; k < 3 * K; ++k) d_sh[(int64_t)k * n + i] = 0.0;
        if (!P.vis) continue;

        const double gu = grads2d[G_U * n + i], gv = grads2d[G_V * n + i];
        const double gA = grads2d[G_A * n + i], gB = grads2d[G_B * n + i], gC = grads2d[G_C * n + i];
        const double go = grads2d[G_O * n + i];
        const double gc[3] = {grads2d[G_R * n + i], grads2d[G_G * n + i], grads2d[G_BL * n + i]};

        /* conic -> Sigma2D */
        const double Q[2][2] = {{P.A, P.B}, {P.B, P.C}};
        const double GQ[2][2] = {{gA, 0.5 * gB}, {0.5 * gB, gC}};
        double QG[2][2], GS2[2][2];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 2; ++c) QG[r][c] = Q[r][0] * GQ[0][c] + Q[r][1] * GQ[1][c];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 2; ++c) GS2[r][c] = -(QG[r][0] * Q[0][c] + QG[r][1] * Q[1][c]);

        /* Sigma2D = T Sigma T^T */
        double GT_[2][3], GSig[3][3], TSig[2][3];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 3; ++c) {
                double acc = 0.0;
                for (int k = 0; k < 3; ++k) acc += P.T[r][k] * P.Sig[k][c];
                TSig[r][c] = acc;
            }
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 3; ++c) GT_[r][c] = 2.0 * (GS2[r][0] * TSig[0][c] + GS2[r][1] * TSig[1][c]);
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) {
                double acc = 0.0;
                for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b) acc += P.T[a][r] * GS2[a][b] * P.T[b][c];
                GSig[r][c] = acc;
            }
        /* T = J W  ->  G_J = G_T W^T */
        double GJ[2][3];
        for (int r = 0; r < 2; ++r)
            for (int c = 0; c < 3; ++c) {
                double acc = 0.0;
                for (int k = 0; k < 3; ++k) acc += GT_[r][k] * cam.R[c][k];
                GJ[r][c] = acc;
            }
        const double X = P.X, Yc = P.Y, Z = P.Z, fx = cam.fx, fy = cam.fy;
        double dp[3] = {0, 0, 0};
        /* J entries: J00 = fx/Z, J02 = -fx X/Z^2, J11 = fy/Z, J12 = -fy Y/Z^2 */
        dp[0] += GJ[0][2] * (-fx / (Z * Z));
        dp[1] += GJ[1][2] * (-fy / (Z * Z));
        dp[2] += GJ[0][0] * (-fx / (Z * Z)) + GJ[0][2] * (2.0 * fx * X / (Z * Z * Z))
               + GJ[1][1] * (-fy / (Z * Z)) + GJ[1][2] * (2.0 * fy * Yc / (Z * Z * Z));
        /* u = fx X/Z + cx, v = fy Y/Z + cy */
        dp[0] += gu * fx / Z;
        dp[1] += gv * fy / Z;
        dp[2] += -gu * fx * X / (Z * Z) - gv * fy * Yc / (Z * Z);
        double dmu[3];
        for (int j = 0; j < 3; ++j) dmu[j] = cam.R[0][j] * dp[0] + cam.R[1][j] * dp[1] + cam.R[2][j] * dp[2];

        /* Sigma = M M^T */
        double GM[3][3];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) {
                double acc = 0.0;
                for (int k = 0; k < 3; ++k) acc += GSig[r][k] * P.M[k][c];
                GM[r][c] = 2.0 * acc;
            }
        for (int k = 0; k < 3; ++k) {
            double ds = 0.0;
            for (int r = 0; r < 3; ++r) ds += GM[r][k] * P.Rq[r][k];
            d_log_scales[k * n + i] = ds * P.s[k];
        }
        double GR[3][3];
        for (int r = 0; r < 3; ++r)
            for (int c = 0; c < 3; ++c) GR[r][c] = GM[r][c] * P.s[c];
        const double w = P.qn[0], x = P.qn[1], y = P.qn[2], z = P.qn[3];
        double dq[4];
        dq[0] = GR[0][1] * (-2 * z) + GR[0][2] * (2 * y) + GR[1][0] * (2 * z) + GR[1][2] * (-2 * x)
              + GR[2][0] * (-2 * y) + GR[2][1] * (2 * x);
        dq[1] = GR[0][1] * (2 * y) + GR[0][2] * (2 * z) + GR[1][0] * (2 * y) + GR[1][1] * (-4 * x)
              + GR[1][2] * (-2 * w) + GR[2][0] * (2 * z) + GR[2][1] * (2 * w) + GR[2][2] * (-4 * x);
        dq[2] = GR[0][0] * (-4 * y) + GR[0][1] * (2 * x) + GR[0][2] * (2 * w) + GR[1][0] * (2 * x)
              + GR[1][2] * (2 * z) + GR[2][0] * (-2 * w) + GR[2][1] * (2 * z) + GR[2][2] * (-4 * y);
        dq[3] = GR[0][0] * (-4 * z) + GR[0][1] * (-2 * w) + GR[0][2] * (2 * x) + GR[1][0] * (2 * w)
              + GR[1][1] * (-4 * z) + GR[1][2] * (2 * y) + GR[2][0] * (2 * x) + GR[2][1] * (2 * y);
        const double qd = P.qn[0] * dq[0] + P.qn[1] * dq[1] + P.qn[2] * dq[2] + P.qn[3] * dq[3];
        for (int j = 0; j < 4; ++j) d_quats[j * n + i] = (dq[j] - P.qn[j] * qd) / P.qnorm;

        /* opacity (the record rounding of o is treated as identity) */
        const double o_exact = 1.0 / (1.0 + exp(-logits[i]));
        d_logits[i] = go * o_exact * (1.0 - o_exact);

        /* colour */
        double vhat[3] = {P.dir[0] / P.dist, P.dir[1] / P.dist, P.dir[2] / P.dist};
        double Ysh[(ORC_MAX_DEG + 1) * (ORC_MAX_DEG + 1)], gY[3 * (ORC_MAX_DEG + 1) * (ORC_MAX_DEG + 1)];
        sh_basis(deg, vhat, Ysh, gY);
        double dv[3] = {0, 0, 0};
        for (int k = 0; k < K; ++k) {
            double kc = 0.0;
            for (int ch = 0; ch < 3; ++ch) {
                d_sh[(int64_t)(k * 3 + ch) * n + i] = Ysh[k] * gc[ch];
                kc += sh[(int64_t)(k * 3 + ch) * n + i] * gc[ch];
            }
            for (int j = 0; j < 3; ++j) dv[j] += kc * gY[3 * k + j];
        }
        const double vd = vhat[0] * dv[0] + vhat[1] * dv[1] + vhat[2] * dv[2];
        for (int j = 0; j < 3; ++j) dmu[j] += (dv[j] - vhat[j] * vd) / P.dist;
        for (int j = 0; j < 3; ++j) d_means[j * n + i] = dmu[j];
    }
    return 0;
}

/* ----------------------------------------------------------------- loss */

/* L1 term of the objective ("Scaling 3D Gaussian Splatting with Distributed
 * Compute", section "Why gsplat Cannot Just Use DDP"; ByteSplat Eq. 2):
 * L = mean over the 3*n_px colour values of |C - C*|, G = sign(C - C*)/(3 n_px)
 * with sign(0) = 0.  reading: mean over all colour elements. */
double orc_loss_l1(int64_t n_px, const float *color, const float *target, double *G)
{
    const int64_t m = 3 * n_px;
    double s = 0.0;
    for (int64_t k = 0; k < m; ++k) {
        const double d = (double)color[k] - (double)target[k];
        s += fabs(d);
        G[k] = (d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0)) / (double)m;
    }
    return m > 0 ? s / (double)m : 0.0;
}

/* ------------------------------------------------------- structural loss */

/*
 * SSIM and the D-SSIM term of the objective.  The pages give the objective
 * ("Scaling 3D Gaussian Splatting with Distributed Compute", section "Why gsplat
 * Cannot Just Use DDP": L = (1 - lambda) L1 + lambda (1 - SSIM(I_r, I_gt)) / 2;
 * Splaxel section 2 "Parameter Optimization": the structural dissimilarity derived
 * from SSIM; ByteSplat Eq. 2) but not the SSIM window or constants.  Reading:
 *   - per colour channel, a (2r+1) x (2r+1) window w(u, v) = g(u) g(v) with
 *     g(u) = exp(-u^2 / (2 sigma^2)) normalised to sum 1 over |u| <= r
 *     (r = 5, sigma = 1.5);
 *   - pixels outside the image count as 0 (zero padding), every window keeps its
 *     full weights;
 *   - at pixel p: mu_x = sum w x, e_xx = sum w x^2, e_xy = sum w x y (and the same
 *     for y), s_xx = e_xx - mu_x^2, s_xy = e_xy - mu_x mu_y,
 *     S(p) = (2 mu_x mu_y + C1)(2 s_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(s_xx + s_yy + C2))
 *     with C1 = 0.01^2, C2 = 0.03^2 (unit dynamic range);
 *   - SSIM = the mean of S over the H W pixels and 3 channels.
 * Images are [H][W][3] float; everything is computed in double by direct sums
 * over each window.  Returns the mean SSIM; smap [H][W][3] (nullable) receives S;
 * grad [H][W][3] (nullable) receives d SSIM / d x (x = the first image), by the
 * chain rule through mu_x, e_xx and e_xy of every window that holds the pixel.
 */
static void ssim_window(int r, double sigma, double *g)
{
    double sum = 0.0;
    for (int u = -r; u <= r; ++u) {
        g[u + r] = exp(-(double)(u * u) / (2.0 * sigma * sigma));
        sum += g[u + r];
    }
    for (int u = -r; u <= r; ++u) g[u + r] /= sum;
}

double orc_ssim(int W, int H, const float *x, const float *y, int r, double sigma, double C1, double C2,
                double *smap, double *grad)
{
    if (W <= 0 || H <= 0 || r < 0 || r > 64) return NAN;
    double g[129];
    ssim_window(r, sigma, g);
    const int64_t np = (int64_t)W * H * 3;
    /* per pixel and channel: dS/dmu_x (total, through s_xx and s_xy too), dS/de_xx, dS/de_xy */
    double *dm = NULL, *dexx = NULL, *dexy = NULL;
    if (grad) {
        dm = (double *)calloc((size_t)np, sizeof(double));
        dexx = (double *)calloc((size_t)np, sizeof(double));
        dexy = (double *)calloc((size_t)np, sizeof(double));
    }
    double total = 0.0;
    for (int py = 0; py < H; ++py)
        for (int px = 0; px < W; ++px)
            for (int c = 0; c < 3; ++c) {
                double mx = 0, my = 0, exx = 0, eyy = 0, exy = 0;
                for (int v = -r; v <= r; ++v)
                    for (int u = -r; u <= r; ++u) {
                        const int qx = px + u, qy = py + v;
                        if (qx < 0 || qx >= W || qy < 0 || qy >= H) continue;   /* zero padding */
                        const double w = g[u + r] * g[v + r];
                        const int64_t q = ((int64_t)qy * W + qx) * 3 + c;
                        const double a = x[q], b = y[q];
                        mx += w * a; my += w * b;
                        exx += w * a * a; eyy += w * b * b; exy += w * a * b;
                    }
                const double sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
                const double n1 = 2.0 * mx * my + C1, n2 = 2.0 * sxy + C2;
                const double d1 = mx * mx + my * my + C1, d2 = sxx + syy + C2;
                const double S = (n1 * n2) / (d1 * d2);
                const int64_t p = ((int64_t)py * W + px) * 3 + c;
                if (smap) smap[p] = S;
                total += S;
                if (grad) {
                    /* partials with mu_x, s_xx, s_xy as independent variables */
                    const double dS_dmx = S * (2.0 * my / n1 - 2.0 * mx / d1);
                    const double dS_dsxx = -S / d2;
                    const double dS_dsxy = 2.0 * S / n2;
                    /* s_xx = e_xx - mu_x^2, s_xy = e_xy - mu_x mu_y */
                    dm[p] = dS_dmx + dS_dsxx * (-2.0 * mx) + dS_dsxy * (-my);
                    dexx[p] = dS_dsxx;
                    dexy[p] = dS_dsxy;
                }
            }
    const double inv = 1.0 / (double)np;
    if (grad) {
        /* d mu_x(p)/d x(q) = w(q - p); d e_xx(p)/d x(q) = 2 w(q - p) x(q); d e_xy(p)/d x(q) = w(q - p) y(q) */
        for (int qy = 0; qy < H; ++qy)
            for (int qx = 0; qx < W; ++qx)
                for (int c = 0; c < 3; ++c) {
                    const int64_t q = ((int64_t)qy * W + qx) * 3 + c;
                    double acc = 0.0;
                    for (int v = -r; v <= r; ++v)
                        for (int u = -r; u <= r; ++u) {
                            const int px = qx - u, py = qy - v;   /* windows centred at p hold q */
                            if (px < 0 || px >= W || py < 0 || py >= H) continue;
                            const double w = g[u + r] * g[v + r];
                            const int64_t p = ((int64_t)py * W + px) * 3 + c;
                            acc += w * (dm[p] + 2.0 * (double)x[q] * dexx[p] + (double)y[q] * dexy[p]);
                        }
                    grad[q] = acc * inv;
                }
        free(dm);
        free(dexx);
        free(dexy);
    }
    return total * inv;
}

/* The objective with both terms ("Scaling 3D Gaussian Splatting with Distributed
 * Compute", "Why gsplat Cannot Just Use DDP"; ByteSplat Eq. 2):
 *   L = (1 - lambda) mean |C - C*| + lambda (1 - SSIM(C, C*)) / 2
 * over the 3 H W colour values, with SSIM as orc_ssim (r = 5, sigma = 1.5,
 * C1 = 0.01^2, C2 = 0.03^2; reading) and sign(0) = 0 in the L1 gradient.
 * G [H][W][3] (nullable) receives dL/dC.  Returns L; *ssim_out (nullable) the SSIM. */
double orc_loss_l1_dssim(int W, int H, const float *color, const float *target, double lambda, double *G,
                         double *ssim_out)
{
    const int64_t np = (int64_t)W * H * 3;
    double *gs = G ? (double *)calloc((size_t)np, sizeof(double)) : NULL;
    const double ssim = orc_ssim(W, H, color, target, 5, 1.5, 1e-4, 9e-4, NULL, gs);
    double l1 = 0.0;
    for (int64_t i = 0; i < np; ++i) {
        const double d = (double)color[i] - (double)target[i];
        l1 += fabs(d);
        if (G) {
            const double sg = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
            G[i] = (1.0 - lambda) * sg / (double)np - 0.5 * lambda * gs[i];
        }
    }
    free(gs);
    if (ssim_out) *ssim_out = ssim;
    return (1.0 - lambda) * l1 / (double)np + lambda * (1.0 - ssim) / 2.0;
}

/* ----------------------------------------------------------------- Adam */

/* Textbook bias-corrected Adam (reading: the pages name Adam with betas
 * (0.9, 0.999) and eps 1e-15 at batch size 1 but not its variant):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p = p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps). */
void orc_adam(int64_t n, const double *p, const double *g, const double *m, const double *v,
              double lr, double b1, double b2, double eps, int step,
              double *p_out, double *m_out, double *v_out)
{
    const double bc1 = 1.0 - pow(b1, step), bc2 = 1.0 - pow(b2, step);
    for (int64_t i = 0; i < n; ++i) {
        const double gi = g[i];
        const double mi = b1 * m[i] + (1.0 - b1) * gi;
        const double vi = b2 * v[i] + (1.0 - b2) * gi * gi;
        p_out[i] = p[i] - lr * (mi / bc1) / (sqrt(vi / bc2) + eps);
        m_out[i] = mi;
        v_out[i] = vi;
    }
}

/* ------------------------------------------------- partial-render compositing */

/* Over-composition of K depth-ordered partial renders (C_k, T_k) along each
 * pixel ray [Splaxel sec. 3.4 and 4.2: partial pixels aggregated along the
 * ray in depth order; convex partitions keep the global blending order]:
 *   A_0 = 1;  for k: if A_k < theta_T the partition is skipped (saturation,
 *   Splaxel sec. 4.3; reading: a skipped partition counts as T_k = 1, C_k = 0),
 *   else C += A_k C_k, A_{k+1} = A_k T_k.  T = A_K. */
void orc_composite(int kparts, int64_t n_px, const float *const *c_k, const float *const *t_k,
                   double t_min, double *c_out, double *t_out)
{
    for (int64_t p = 0; p < n_px; ++p) {
        double A = 1.0, C[3] = {0, 0, 0};
        for (int k = 0; k < kparts; ++k) {
            if (A < t_min) continue;
            for (int ch = 0; ch < 3; ++ch) C[ch] += A * (double)c_k[k][3 * p + ch];
            A *= (double)t_k[k][p];
        }
        for (int ch = 0; ch < 3; ++ch) c_out[3 * p + ch] = C[ch];
        t_out[p] = A;
    }
}

/* Backward of orc_composite (no division):
 *   dL/dC_k = A_k G
 *   dL/dT_k = A_k (U_k . G) + (prod_{m != k} T_m) G_T,
 *   U_k = C_{k+1} + T_{k+1} U_{k+1} (the composite behind k), U_last = 0;
 * skipped partitions get zero gradients. */
void orc_composite_bwd(int kparts, int64_t n_px, const float *const *c_k, const float *const *t_k,
                       double t_min, const double *G, const double *GT,
                       double *const *dc_k, double *const *dt_k)
{
    double A[64], U[64][3], S[65];
    int act[64];
    for (int64_t p = 0; p < n_px; ++p) {
        double a = 1.0;
        for (int k = 0; k < kparts; ++k) {
            A[k] = a;
            act[k] = !(a < t_min);
            if (act[k]) a *= (double)t_k[k][p];
        }
        /* suffix composites and suffix transmittance products over active partitions */
        double u[3] = {0, 0, 0};
        S[kparts] = 1.0;
        for (int k = kparts - 1; k >= 0; --k) {
            for (int ch = 0; ch < 3; ++ch) U[k][ch] = u[ch];
            if (act[k]) {
                for (int ch = 0; ch < 3; ++ch) u[ch] = (double)c_k[k][3 * p + ch] + (double)t_k[k][p] * u[ch];
                S[k] = S[k + 1] * (double)t_k[k][p];
            } else {
                S[k] = S[k + 1];
            }
        }
        const double gt = GT ? GT[p] : 0.0;
        for (int k = 0; k < kparts; ++k) {
            if (!act[k]) {
                for (int ch = 0; ch < 3; ++ch) dc_k[k][3 * p + ch] = 0.0;
                dt_k[k][p] = 0.0;
                continue;
            }
            for (int ch = 0; ch < 3; ++ch) dc_k[k][3 * p + ch] = A[k] * G[3 * p + ch];
            const double ug = U[k][0] * G[3 * p] + U[k][1] * G[3 * p + 1] + U[k][2] * G[3 * p + 2];
            dt_k[k][p] = A[k] * ug + A[k] * S[k + 1] * gt;
        }
    }
}

/* ------------------------------------------------------- gradient records */

/* Zero-gradient elision [ByteSplat sec. 3 Insight 4, sec. 6]: a Gaussian's
 * screen-space partial gradient is dropped when all of its fields are exactly
 * zero (-0.0 compares equal to zero).  Records {uint32 index_base + i,
 * float g[9]} are written in ascending index order; bitmap bit (i mod 32) of
 * word i/32 is set for kept records.  Returns the record count. */
int64_t orc_compact(int64_t n, const float *grads2d, uint32_t index_base,
                    uint32_t *records /* [R][10] */, uint32_t *bitmap)
{
    const int64_t words = (n + 31) / 32;
    memset(bitmap, 0, sizeof(uint32_t) * (size_t)words);
    int64_t r = 0;
    for (int64_t i = 0; i < n; ++i) {
        int nz = 0;
        for (int f = 0; f < 9; ++f)
            if (grads2d[f * n + i] != 0.0f) nz = 1;
        if (!nz) continue;
        bitmap[i / 32] |= 1u << (i % 32);
        records[10 * r] = index_base + (uint32_t)i;
        for (int f = 0; f < 9; ++f) memcpy(&records[10 * r + 1 + f], &grads2d[f * n + i], 4);
        ++r;
    }
    return r;
}

/* Owner-side aggregation of compacted records [ByteSplat sec. 6.2, Fig. 9]:
 * every record of partition k names a partition position i = index - base[k];
 * the forward-communication index maps it to the owner's Gaussian
 * o = owner_index[k][i] (identity when that array is NULL), and the record's
 * nine fields are added to field planes out[f][o] (accumulated, double).
 * Records whose position or owner Gaussian is out of range are skipped and
 * counted; the count is returned. */
int64_t orc_decode(int k, const uint32_t *const *records, const int64_t *r, const uint32_t *base,
                   const uint32_t *const *owner_index, const int64_t *n_part, int64_t n_owner,
                   double *out /* [9][n_owner] */)
{
    int64_t rejected = 0;
    for (int q = 0; q < k; ++q) {
        for (int64_t j = 0; j < r[q]; ++j) {
            const uint32_t *rec = records[q] + 10 * j;
            const int64_t i = (int64_t)rec[0] - (int64_t)base[q];
            if (i < 0 || i >= n_part[q]) {
                ++rejected;
                continue;
            }
            const int64_t o = owner_index[q] ? (int64_t)owner_index[q][i] : i;
            if (o >= n_owner) {
                ++rejected;
                continue;
            }
            for (int f = 0; f < 9; ++f) {
                float v;
                memcpy(&v, &rec[1 + f], 4);
                out[f * n_owner + o] += (double)v;
            }
        }
    }
    return rejected;
}

/* Adam hyper-parameters for BS views per optimiser step ["Scaling 3D Gaussian Splatting
 * with Distributed Compute", section "Batching and Hyperparameter Scaling"]: learning
 * rates grow with the square root of BS, eps shrinks by it, and each momentum coefficient
 * is linearised as 1 - BS (1 - beta).  lr: 6 rates in, scaled in place.  Returns 0, or -1
 * when a scaled beta leaves [0, 1). */
int orc_adam_batch_hparams(int bs, double *lr, double *beta1, double *beta2, double *eps)
{
    const double root = sqrt((double)bs);
    const double b1 = 1.0 - bs * (1.0 - *beta1), b2 = 1.0 - bs * (1.0 - *beta2);
    if (bs < 1 || !(b1 >= 0.0 && b1 < 1.0 && b2 >= 0.0 && b2 < 1.0)) return -1;
    for (int a = 0; a < 6; ++a) lr[a] *= root;
    *beta1 = b1;
    *beta2 = b2;
    *eps /= root;
    return 0;
}
