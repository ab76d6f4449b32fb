/*
 * gs.h -- C ABI of libgsmi, the one-GPU 3D Gaussian splatting training step
 * for AMD Instinct MI355X (gfx950).
 *
 * The step, as the sources describe it (page titles; sections / equations):
 *   projection + SH colour  -> gs_project     "Splaxel: Efficient Distributed Training of 3D
 *                                             Gaussian Splatting for Large-scale Scene
 *                                             Reconstruction via Pixel-level Communication",
 *                                             section 2 ("Projection"); "Scaling 3D Gaussian
 *                                             Splatting with Distributed Compute" (ROCm blog),
 *                                             walkthrough steps 3-4
 *   tile binning + depth sort -> gs_bin_sort  "ByteSplat: Efficient Distributed 3D Gaussian
 *                                             Splatting Training via Intra- and Inter-GPU
 *                                             communication reduction", section 2.1
 *                                             ("Projection", "Sorting")
 *   front-to-back compositing -> gs_raster_fwd  ByteSplat section 2.1, Eq. 1
 *   L1 loss                   -> gs_loss_l1      ByteSplat Eq. 2 (L1 term); ROCm blog, loss
 *   L1 + D-SSIM loss          -> gs_loss_l1_dssim  ROCm blog, loss; Splaxel section 2
 *   backward rasterization    -> gs_raster_bwd   ByteSplat section 2.1, Eq. 3 and Eq. 4, then
 *                                                the backward through projection and colour
 *   parameter update          -> gs_adam_step    ROCm blog, create_splats_with_optimizers
 *   partial renders of depth slabs, their over-composition and the compaction of non-zero
 *   gradient records -> gs_composite_over(_bwd), gs_compact_grads  (Splaxel sections 4.2-4.3;
 *   ByteSplat section 3 Insight 4 and section 6.1)
 *   owner-side decoding and atomic aggregation of those records -> gs_decode_grads
 *   (ByteSplat section 6.2); the owner's update from the decoded gradients ->
 *   gs_project_bwd_adam
 *   batches of views per optimiser step -> gs_project_batch, gs_grad_aggregate_adam_batch,
 *   gs_adam_batch_hparams  (ROCm blog, "Batching and Hyperparameter Scaling")
 *
 * Conventions (all entry points):
 *   - Every pointer argument that names device memory must be a device (or managed)
 *     allocation owned by the caller; the library never allocates or frees memory.
 *     Host pointers are marked "host".
 *   - All calls enqueue work on `stream` and return without waiting, except where a
 *     function says it reads a count back to the host (it then synchronises `stream`).
 *   - Arrays are float32/int32 unless stated; "[a][b]" is row-major (b fastest).
 *   - Errors: arguments are checked on the host before anything is launched; a non-OK
 *     status leaves outputs unspecified and gs_last_error() describes the problem.
 *     HIP runtime failures return GS_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Thread safety: calls are reentrant; the only global state is the thread-local
 *     error message.  Calls on different streams may run concurrently if their
 *     buffers do not overlap.
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, negative size, bad image size ... */
    GS_ERR_UNSUPPORTED = 2,      /* e.g. SH degree > 3, more tiles than the sort supports */
    GS_ERR_CAPACITY = 3,         /* an output list is too small; the required size is reported */
    GS_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} gs_status;

#define GS_TILE 16          /* tiles are 16x16 pixels (ByteSplat section 2.2) */
#define GS_MAX_SH_DEGREE 3
#define GS_RADIUS_CAP (1 << 20)

/* Pinhole camera, OpenCV axes (x right, y down, z forward).  viewmat is the
 * row-major 4x4 world->camera matrix (rows 0..2 = [R | t]); pixel (i, j) has its
 * centre at (i + 0.5, j + 0.5). */
typedef struct {
    float viewmat[16];
    float fx, fy, cx, cy;
    int32_t width, height;   /* 1 .. 65536, at most 2^24 tiles */
    float near_z;            /* Gaussians with camera depth <= near_z are culled */
} gs_camera;

typedef struct {
    int32_t sh_degree;  /* 0..3: (sh_degree+1)^2 coefficients per colour channel */
    float alpha_min;    /* alpha-check: entries with alpha < alpha_min are skipped (1/255) */
    float alpha_max;    /* alpha is clamped to at most alpha_max (0.99); must be < 1 */
    float t_min;        /* compositing stops before an entry once T < t_min (1e-4); 0 disables */
    float depth_lo;     /* only Gaussians whose depth key d satisfies depth_lo <= d < depth_hi */
    float depth_hi;     /*   are projected (depth slab of a partial render); 0, +inf = all */
} gs_raster_params;

/* Learnable parameters, structure of arrays (planes of n floats):
 *   means [3][n], log_scales [3][n] (scale = exp), quats [4][n] (w, x, y, z; normalised
 *   in the forward), opacity_logits [n] (opacity = sigmoid), sh [K*3][n] with
 *   K = (sh_degree+1)^2 and plane k*3 + c holding coefficient k of channel c
 *   (k = l*l + l + m, real orthonormal basis without Condon-Shortley phase).
 * ld: floats from one plane of a group to the next, the same for every group (0: n;
 *   otherwise >= n).  Plane f of means is means[f * ld .. f * ld + n).  The kernels read
 *   and write one plane segment per 64 Gaussians: with ld a multiple of 32 every segment
 *   of a 256-byte-aligned group covers whole 128-byte lines; otherwise most segments
 *   straddle lines that neighbouring waves write too, which on MI355X costs the
 *   per-Gaussian passes up to twice their time (a padded ld of 64 is the recommended
 *   layout). */
typedef struct {
    const float *means, *log_scales, *quats, *opacity_logits, *sh;
    int64_t n;
    int64_t ld;
} gs_gaussians;

/* Projected 2D records, one per Gaussian.
 *   depth [n]             camera-space depth as a float32 key:
 *                         fma(R22, z, fma(R21, y, R20 * x)) + t2, each step rounded
 *   radii [n][2]          half-extents in pixels of the alpha >= alpha_min ellipse box,
 *                         rounded up, >= 1; (0, 0) marks a culled Gaussian (8-byte aligned)
 *   rec [n][12]           the raster record (16-byte aligned): u, v (pixel coordinates of
 *                         the mean), the conic pre-scaled for a base-2 exponential
 *                         (-A log2(e)/2, -B log2(e), -C log2(e)/2), log2(o), red, green,
 *                         blue, the index as uint32 bits, rx and ry as int32 bits.
 *                         gs_bin_sort takes each Gaussian's tile box and quadrant test from
 *                         it and the raster entry points read it.  A culled Gaussian's
 *                         record is zero apart from its index.
 * Optional plain copies of the same record, planes of n floats; each pointer may be NULL,
 * and then that group is not written:
 *   means2d [2][n]        u, v
 *   conic_opacity [4][n]  A, B, C, o: inverse 2D covariance [[A, B], [B, C]] and opacity
 *   color [3][n]          RGB from the SH coefficients (no offset, no clamp)
 * They are written for visible Gaussians only. */
typedef struct {
    float *means2d, *conic_opacity, *color, *depth;
    int32_t *radii;
    float *rec;
} gs_projected;

/* Tile-Gaussian intersection lists.
 *   ids [capacity]            Gaussian index of each entry, sorted by (tile, depth key, index)
 *   tile_ranges [tiles + 1]   entries of tile t are ids[tile_ranges[t] .. tile_ranges[t+1])
 *   keys [capacity]           optional (may be NULL): tile << 32 | depth key bits per entry
 *   tiles_touched [n]         optional (may be NULL): number of tiles of each Gaussian
 *   raster                    gs_bins_raster_bytes(n, capacity, W, H) bytes of device memory,
 *                             256-byte aligned, written by gs_bin_sort and read (and, for the
 *                             per-record gradient slots, written) by the raster entry points:
 *                             for each 8x8 quadrant of every tile, the records of the tile's
 *                             entries whose box reaches it, the maps the backward needs to sum
 *                             each Gaussian's contributions, and the order in which tiles are
 *                             rasterized.  Its layout is private to the library; the caller
 *                             only owns the memory, which may be uninitialised (fresh or
 *                             reused) before the first gs_bin_sort: the sort writes
 *                             everything the raster calls read, including the stamps that
 *                             mark which gradient slots a backward call has written.  The
 *                             raster calls must use the same n, capacity and image size as
 *                             the gs_bin_sort call that filled it.
 * tiles = ceil(W/16) * ceil(H/16), tile id = row * ceil(W/16) + column; capacity <= 2^30. */
typedef struct {
    uint32_t *ids;
    int32_t *tile_ranges;
    uint64_t *keys;
    int32_t *tiles_touched;
    int64_t capacity;
    void *raster;
} gs_bins;

/* Gradients of the learnable parameters (or Adam moments), same shapes as gs_gaussians;
 * ld: their plane stride (0: the Gaussians' n; otherwise >= n). */
typedef struct {
    float *means, *log_scales, *quats, *opacity_logits, *sh;
    int64_t ld;
} gs_param_grads;

/* One Adam parameter group: n scalars of parameters p, gradients g, moments m, v. */
typedef struct {
    float *p;
    const float *g;
    float *m, *v;
    int64_t n;
    float lr;
} gs_adam_group;

/* Projection and colour evaluation, one thread per Gaussian (Splaxel section 2:
 * Sigma = R S S^T R^T, frustum culling by the mean, Sigma2D = J W Sigma W^T J^T;
 * ROCm blog step 4: SH evaluated to RGB per camera).  Culls a Gaussian if an input is
 * not finite, |q| = 0, its depth key is outside [depth_lo, depth_hi), its camera depth
 * is <= near_z, its projected mean lies outside [0, W) x [0, H), det(Sigma2D) <= 0, or
 * its opacity < alpha_min.  The geometric chain runs in double and is rounded to
 * the float32 record.  Inputs: g (n >= 0), cam, p.  Outputs: out (n records). */
gs_status gs_project(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                     gs_projected *out, hipStream_t stream);

/* Bytes of the gs_bins.raster buffer for n Gaussians, `capacity` list entries and a W x H
 * image: 2 quadrant entries (12 B), 2 gradient slots (48 B) with their stamps (4 B) and 4
 * quadrant bits per entry, plus 68 B per Gaussian (a copy of its 48-byte raster record at a
 * 64-byte stride and its first gradient slot), 16 B per tile and a 256-byte header. */
size_t gs_bins_raster_bytes(int64_t n, int64_t capacity, int32_t width, int32_t height);

/* Workspace bytes gs_bin_sort needs for n Gaussians, `capacity` list entries and the
 * camera's image size. */
size_t gs_bin_sort_workspace_bytes(int64_t n, int64_t capacity, int32_t width, int32_t height);

/* Tile binning and depth sort (ByteSplat section 2.1, "Projection" and "Sorting").
 * Every Gaussian with radii > 0 emits one entry per 16x16 tile its box
 * [u - rx, u + rx] x [v - ry, v + ry] touches (float32 arithmetic:
 * x0 = clamp(floor((u - rx)/16), 0, TX), x1 = clamp(floor((u + rx)/16) + 1, 0, TX), same
 * for y).  Entries are ordered by (tile, depth key bits, Gaussian index): a stable LSD
 * radix sort of the Gaussians by depth key, a scan of their tile counts in that order,
 * emission, and a stable radix sort of the entries by tile id.  Then fills bins->raster
 * from the projected records (proj->depth, radii and rec are read; u, v, rx, ry as stored in
 * rec; the records themselves are copied in): an entry joins the list of an 8x8 quadrant
 * of its tile if its alpha >= p->alpha_min ellipse can reach one of the quadrant's pixel
 * centres.  p must be the parameters given
 * to gs_project.
 * Reads the total K back to the host (synchronises `stream`) and stores it in
 * *n_isect_out (host).  The quadrant records take up to 2 * capacity slots, so a capacity
 * below max(K, ceil(Q / 2)) (Q = the number of (entry, quadrant) pairs) returns
 * GS_ERR_CAPACITY with that required capacity in *n_isect_out and the lists unspecified.  workspace: device memory of at least
 * gs_bin_sort_workspace_bytes(n, capacity, W, H) bytes, 256-byte aligned. */
gs_status gs_bin_sort(const gs_projected *proj, int64_t n, const gs_camera *cam, const gs_raster_params *p,
                      gs_bins *bins, int64_t *n_isect_out, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* gs_bin_sort without the read-back: nothing in the call waits for the device, so a
 * training step can be queued (or captured) as a whole.  Every launch after the counting is
 * sized by bins->capacity and reads the entry count on the device.  counts (device, may be
 * NULL, 8-byte aligned): receives {K, required capacity} as two int64 when the stream gets
 * there; required capacity is 0 when the lists fit, else the capacity gs_bin_sort would
 * report with GS_ERR_CAPACITY.  Lists that do not fit are left empty (every tile range
 * empty; gs_raster_fwd then renders nothing and gs_raster_bwd / gs_grad_aggregate write zero
 * gradients): the caller checks counts, grows the buffers and repeats the step.  Otherwise
 * identical results to gs_bin_sort. */
gs_status gs_bin_sort_async(const gs_projected *proj, int64_t n, const gs_camera *cam, const gs_raster_params *p,
                            gs_bins *bins, int64_t *counts, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Front-to-back alpha compositing per 16x16 tile (ByteSplat Eq. 1): for each pixel,
 * T = 1; for each entry of its tile list in order: stop if T < t_min; alpha =
 * min(alpha_max, o exp(-A dx^2/2 - B dx dy - C dy^2/2)); skip if alpha < alpha_min;
 * C += T alpha c; T *= 1 - alpha.  Outputs color [H][W][3], t_final [H][W] (T after the
 * last accepted entry) and n_trav [H][W] (number of list entries the pixel traversed,
 * N_p of Eq. 1).  If n_trav_sum (device, may be NULL) is given, sum_p N_p -- the number of
 * Gaussian-pixel evaluations -- is added to it (the caller clears it).  No background is
 * added. */
gs_status gs_raster_fwd(const gs_projected *proj, const gs_bins *bins, const gs_camera *cam,
                        const gs_raster_params *p, float *color, float *t_final, int32_t *n_trav,
                        unsigned long long *n_trav_sum, hipStream_t stream);

/* Workspace bytes gs_loss_l1 needs for n_px pixels. */
size_t gs_loss_workspace_bytes(int64_t n_px);

/* L1 term of the loss (ByteSplat Eq. 2): loss = mean over the 3*n_px colour values of
 * |color - target|; dL_dcolor = sign(color - target) / (3 n_px) with sign(0) = 0.
 * loss_out: device float (may be NULL); dL_dcolor [n_px][3].  The sum is accumulated in
 * double.  workspace: gs_loss_workspace_bytes(n_px) bytes of device memory. */
gs_status gs_loss_l1(const float *color, const float *target, int64_t n_px, float *loss_out,
                     float *dL_dcolor, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The objective with its structural term (ROCm blog, "Why gsplat Cannot Just Use DDP":
 * L = (1 - lambda) mean |C - C*| + lambda (1 - SSIM(C, C*)) / 2 over the 3 W H colour
 * values; Splaxel section 2 "Parameter Optimization"; ByteSplat Eq. 2) and dL/dC.  The
 * pages fix neither the SSIM window nor its constants; this library reads them as: per
 * colour channel, an 11 x 11 Gaussian window (sigma 1.5, normalised over its support),
 * zero padding outside the image, C1 = 0.01^2, C2 = 0.03^2, SSIM = the mean over pixels
 * and channels of S = (2 mu_x mu_y + C1)(2 s_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(s_xx + s_yy
 * + C2)); sign(0) = 0 in the L1 term.  color, target, dL_dcolor: [H][W][3]; 0 <= lambda
 * <= 1 (lambda = 0 is gs_loss_l1's objective); loss_out, ssim_out: device floats (each may
 * be NULL), the sums taken in double in a fixed order.  workspace:
 * gs_loss_l1_dssim_workspace_bytes(W, H) bytes (256-byte aligned): three coefficient maps
 * per channel (36 B per pixel) and per-tile partial sums.  Images of 12 W H >= 2^32 bytes
 * (the kernels index in 32 bits) return GS_ERR_UNSUPPORTED, and their workspace size is 0. */
size_t gs_loss_l1_dssim_workspace_bytes(int32_t width, int32_t height);
gs_status gs_loss_l1_dssim(const float *color, const float *target, int32_t width, int32_t height, float lambda,
                           float *loss_out, float *ssim_out, float *dL_dcolor, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Backward rasterization (ByteSplat Eq. 3 and Eq. 4): per tile, each pixel walks its
 * traversed entries front to back, recomputing T_i as the forward pass did, takes the
 * colour composited behind entry i from the forward pass's final colour (T_i B_i (1 -
 * alpha_i) = C - sum_{j<=i} T_j alpha_j c_j), and forms its partial gradient of the
 * Gaussian's 9 screen-space fields, in the order (u, v, A, B, C, o, r, g, b) of grads2d
 * [9][n].  The partial gradients are summed per tile quadrant and then per Gaussian in a
 * fixed order (no atomics): repeated calls give bit-identical results.  Every entry of
 * grads2d is written (zero for culled Gaussians).  dL_dcolor [H][W][3]; dL_dt [H][W] is
 * the gradient of t_final (may be NULL).  color, t_final and n_trav come from
 * gs_raster_fwd on the same inputs.  If grads3d is non-NULL the aggregated screen-space
 * gradients are then propagated through projection and colour evaluation into grads3d
 * (every entry overwritten; zero for culled Gaussians). */
gs_status gs_raster_bwd(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                        const gs_camera *cam, const gs_raster_params *p, const float *color,
                        const float *t_final, const int32_t *n_trav, const float *dL_dcolor, const float *dL_dt,
                        float *grads2d, gs_param_grads *grads3d, hipStream_t stream);

/* The two halves of gs_raster_bwd, for callers that time or schedule them separately;
 * gs_raster_bwd is gs_raster_bwd_partials followed by gs_grad_aggregate on the same
 * stream.  gs_raster_bwd_partials: ByteSplat Eq. 3 per pixel and the per-quadrant part of
 * the Eq. 4 sum, written to per-record slots inside bins->raster (nothing outside it is
 * written; same arguments and checks as gs_raster_bwd).  The slots hold per-record sums of
 * pixel moments, stamped with a counter the call advances, so gs_grad_aggregate reads only
 * the slots of the latest gs_raster_bwd_partials call on these bins.  gs_grad_aggregate: the
 * per-Gaussian part of the Eq. 4 sum over those slots,
 * turned into the screen-space gradients with the Gaussian's conic and opacity from
 * proj->rec, into grads2d [9][n] (every entry written), then, if grads3d is non-NULL, the
 * projection backward as in gs_raster_bwd.  Between the two calls the bins must not be
 * re-sorted; proj is the gs_project output the bins were sorted from. */
gs_status gs_raster_bwd_partials(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam,
                                 const gs_raster_params *p, const float *color, const float *t_final,
                                 const int32_t *n_trav, const float *dL_dcolor, const float *dL_dt,
                                 hipStream_t stream);
gs_status gs_grad_aggregate(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                            const gs_camera *cam, const gs_raster_params *p, float *grads2d,
                            gs_param_grads *grads3d, hipStream_t stream);

/* Forward rasterization, L1 loss and the per-record part of the backward in one kernel
 * (ByteSplat section 4.2, "Fused Rasterization Dataflow"): each 8x8 quadrant composites its
 * pixels (Eq. 1), forms dL/dC = sign(C - target) / (3 W H) per channel at once (the L1 term
 * of Eq. 2, tile-local) and runs the backward walk of Eq. 3 from registers, so the image,
 * N_p and dL/dC are not read back.  Equal, bit for bit, to gs_raster_fwd, gs_loss_l1 and
 * gs_raster_bwd_partials (without dL/dT) in sequence: color [H][W][3], t_final [H][W] and
 * n_trav [H][W] are written as by gs_raster_fwd, and the gradient slots in bins->raster as by
 * gs_raster_bwd_partials (follow with gs_grad_aggregate or gs_grad_aggregate_adam(_project)).
 * target [H][W][3]: the reference image.  loss_out (device, may be NULL): the mean of
 * |C - target|, equal to gs_loss_l1's up to the order of its double-precision sum.
 * n_trav_sum (device, may be NULL): sum_p N_p is added to it, as in gs_raster_fwd.
 * walk_counts (device, may be NULL, 8-byte aligned, 3 x uint64): when given, the call runs a
 * counting instance of the same kernel, which also adds, over all 8x8 quadrant waves, the
 * number of records the forward walk evaluated, the number the backward walk evaluated
 * (each record is evaluated for the wave's 64 pixels, those outside the image included) and
 * the number of (pixel, record) pairs the forward accepted (alpha-check passed before
 * termination); its results are otherwise identical.  It costs one more vector instruction
 * per pair, so timed calls pass NULL.
 * workspace: gs_raster_fused_l1_workspace_bytes(W, H) bytes (16-byte aligned) of per-wave
 * partial sums.  Every tile takes this path: records stream through registers in batches,
 * so no tile is too large for it. */
size_t gs_raster_fused_l1_workspace_bytes(int32_t width, int32_t height);
gs_status gs_raster_fused_l1(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam,
                             const gs_raster_params *p, const float *target, float *color, float *t_final,
                             int32_t *n_trav, float *loss_out, unsigned long long *n_trav_sum,
                             unsigned long long *walk_counts, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* gs_raster_fused_l1 for callers that cannot allocate device memory or be handed a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the per-wave partial sums in a
 * file-scope device array of the library (GS_FUSED_NOALLOC_MAX_WAVES quadrant waves,
 * i.e. images of up to 4096 x 4096 pixels; about 4 MiB held by each GPU the library runs
 * on until the process ends).  Calls no allocation routine.  Larger images return
 * GS_ERR_UNSUPPORTED.  Every call on one GPU uses that GPU's one array: calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised by the caller.
 * The array's contents are not needed between calls (each call rewrites what it reads). */
#define GS_FUSED_NOALLOC_MAX_WAVES (256 * 256 * 4)
gs_status gs_raster_fused_l1_noalloc(const gs_gaussians *g, const gs_bins *bins, const gs_camera *cam,
                                     const gs_raster_params *p, const float *target, float *color, float *t_final,
                                     int32_t *n_trav, float *loss_out, unsigned long long *n_trav_sum,
                                     unsigned long long *walk_counts, hipStream_t stream);

/* Tile budget diagnostic (ByteSplat section 5.2, Eq. 7-9).  gs_tile_budget: B =
 * floor((lds_budget_bytes - fixed_bytes) / bytes_per_gaussian), the number of Gaussian
 * records a tile can keep on chip in a design that holds them there (Eq. 7); -1 for
 * invalid arguments.  gs_tile_budget_report: for the tile lists in bins, per tile t with
 * N_t entries, excess[t] = E_t = max(0, N_t - budget) (Eq. 8) and frac[t] = P_t = E_t / N_t,
 * 0 for an empty tile (Eq. 9) (each may be NULL; tiles-long arrays); totals (device, may be
 * NULL, 8-byte aligned): totals[0] += the number of tiles with E_t > 0, totals[1] += sum_t
 * E_t.  The fused kernel above needs no budget (it streams); the report says how tiles
 * would fare in one that does. */
int64_t gs_tile_budget(int64_t lds_budget_bytes, int64_t fixed_bytes, int64_t bytes_per_gaussian);
gs_status gs_tile_budget_report(const gs_bins *bins, const gs_camera *cam, int64_t budget, int32_t *excess,
                                float *frac, unsigned long long *totals, hipStream_t stream);

/* Learning rates of the fused step below, per parameter group (the SH coefficients split
 * into the DC term, planes 0..2, and the rest). */
typedef struct {
    float means, log_scales, quats, opacity_logits, sh_dc, sh_rest;
} gs_adam_lrs;

/* The end of a training step in one pass over the Gaussians, for callers that update
 * right after each backward (batch size 1): per Gaussian, the per-Gaussian part of the
 * ByteSplat Eq. 4 sum (as gs_grad_aggregate), the projection backward (as gs_project_bwd)
 * and the Adam update of every parameter scalar (as gs_adam_step with the groups means,
 * log_scales, quats, opacity_logits, sh planes 0..2, sh planes 3.., and the learning rates
 * in lr).  The 3D gradients are never stored.  The results equal gs_grad_aggregate,
 * gs_project_bwd and gs_adam_step in sequence, bit for bit.  g: the parameters, read and
 * then updated in place (the arrays must be writable device memory).  m, v: the Adam
 * moments, same shapes as the parameters, updated in place.  grads2d [9][n] (may be NULL):
 * receives the screen-space gradients.  bins, cam, p: as for gs_grad_aggregate. */
gs_status gs_grad_aggregate_adam(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                                 const gs_camera *cam, const gs_raster_params *p, float *grads2d,
                                 const gs_param_grads *m,
                                 const gs_param_grads *v, const gs_adam_lrs *lr, int32_t step, float beta1,
                                 float beta2, float eps, hipStream_t stream);

/* gs_grad_aggregate_adam, then the projection of the updated Gaussians for the camera of
 * the next step, in the same pass: each Gaussian is projected from the updated values the
 * Adam update leaves in registers, so the parameters are not read a second time.  The
 * step that follows starts at gs_bin_sort.  next_proj receives exactly what
 * gs_project(g, next_cam, p, next_proj) would write after gs_grad_aggregate_adam (Splaxel
 * section 2 "Projection", with the same p); it may be the same buffers as proj, which this
 * call does not read.  next_cam must not be NULL.  Errors as gs_grad_aggregate_adam and
 * gs_project. */
gs_status gs_grad_aggregate_adam_project(const gs_gaussians *g, const gs_projected *proj, const gs_bins *bins,
                                         const gs_camera *cam, const gs_raster_params *p, float *grads2d,
                                         const gs_param_grads *m, const gs_param_grads *v, const gs_adam_lrs *lr,
                                         int32_t step, float beta1, float beta2, float eps,
                                         const gs_camera *next_cam, gs_projected *next_proj, hipStream_t stream);

/* ---- batches of views (ROCm blog, "Batching and Hyperparameter Scaling": several camera
 * views per optimiser step; gsplat's projection of C cameras x N Gaussians in one call).
 * A batch holds 1 <= views <= 4 views; cams, bins, out and next_proj are host arrays of
 * `views` structs. */

/* Projects the Gaussians for every camera of the batch in one pass over the parameters:
 * out[k] receives exactly what gs_project(g, &cams[k], p, &out[k]) writes. */
gs_status gs_project_batch(const gs_gaussians *g, int32_t views, const gs_camera *cams,
                           const gs_raster_params *p, gs_projected *out, hipStream_t stream);

/* The end of a training step over a batch of views in one pass over the Gaussians: per
 * Gaussian and for k = 0 .. views-1 in order, the per-Gaussian part of the ByteSplat Eq. 4
 * sum over the slots of bins[k] (written by gs_raster_bwd_partials or gs_raster_fused_l1
 * for camera cams[k]), its screen-space gradients multiplied by grad_scale (1/views for the
 * mean of the views' losses), and the projection backward for cams[k], added to the 3D
 * gradients of the views before it; then one Adam update with the sum (as
 * gs_grad_aggregate_adam); then, if next_cams is non-NULL, the projection of the updated
 * Gaussian for every next_cams[k] into next_proj[k] (as gs_project_batch).  For a
 * power-of-two grad_scale the result equals, bit for bit, gs_grad_aggregate and
 * gs_project_bwd per view, the 3D gradients scaled by grad_scale and added in view order,
 * and gs_adam_step.  The 3D gradients are never stored.  Adam hyper-parameters for a batch:
 * gs_adam_batch_hparams. */
gs_status gs_grad_aggregate_adam_batch(const gs_gaussians *g, int32_t views, const gs_bins *bins,
                                       const gs_camera *cams, const gs_raster_params *p, float grad_scale,
                                       const gs_param_grads *m, const gs_param_grads *v, const gs_adam_lrs *lr,
                                       int32_t step, float beta1, float beta2, float eps,
                                       const gs_camera *next_cams, gs_projected *next_proj, hipStream_t stream);

/* Adam hyper-parameters for a batch of `batch` views (ROCm blog, "Batching and
 * Hyperparameter Scaling", with BS = batch on one GPU): every learning rate times
 * sqrt(BS), eps / sqrt(BS), beta_i -> 1 - BS (1 - beta_i), in double precision and rounded
 * to float once.  Host only (no device work).  GS_ERR_INVALID_ARGUMENT if batch < 1 or a
 * scaled beta falls outside [0, 1) (beta1 = 0.9 reaches 0 at BS = 10). */
gs_status gs_adam_batch_hparams(int32_t batch, double beta1, double beta2, double eps, const gs_adam_lrs *lr,
                                gs_adam_lrs *lr_out, float *beta1_out, float *beta2_out, float *eps_out);

/* Backward through projection and colour evaluation alone (ByteSplat section 2.1: the
 * aggregated screen-space gradients are propagated through projection and colour
 * evaluation): from grads2d [9][n] (fields u, v, A, B, C, o, r, g, b) to grads3d (every
 * entry overwritten; zero for Gaussians the projection culls).  Same g, cam and p as the
 * gs_project call that produced the records.  Lets the caller aggregate screen-space
 * gradients from several partial renders before one projection backward. */
gs_status gs_project_bwd(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                         const float *grads2d, gs_param_grads *grads3d, hipStream_t stream);

/* Bias-corrected Adam over up to 16 parameter groups in one launch (ROCm blog,
 * create_splats_with_optimizers: eps 1e-15, betas (0.9, 0.999) at batch size 1):
 * m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; p -= lr (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps).
 * step t >= 1.  The gradients are read, not modified. */
gs_status gs_adam_step(const gs_adam_group *groups, int32_t n_groups, int32_t step, float beta1,
                       float beta2, float eps, hipStream_t stream);

/* Over-composition of k depth-ordered partial renders along each pixel ray (Splaxel
 * sections 3.4 and 4.2; saturation skip of section 4.3): A = 1, C = 0; for each partition:
 * if A < t_min it is skipped, else C += A C_k and A *= T_k.  t_out = A.
 * c_k: host array of k device pointers to [n_px][3]; t_k: host array of k pointers to
 * [n_px]; 1 <= k <= 16. */
gs_status gs_composite_over(const float *const *c_k, const float *const *t_k, int32_t k,
                            int64_t n_px, float t_min, float *c_out, float *t_out,
                            hipStream_t stream);

/* Backward of gs_composite_over: dL/dC_k = A_k dL/dC; dL/dT_k = A_k (U_k . dL/dC) +
 * (prod_{m != k} T_m) dL/dT with U_k the composite of the partitions behind k; skipped
 * partitions get zeros.  dL_dt may be NULL.  dL_dc_k / dL_dt_k: host arrays of k device
 * pointers. */
gs_status gs_composite_over_bwd(const float *const *c_k, const float *const *t_k, int32_t k,
                                int64_t n_px, float t_min, const float *dL_dc, const float *dL_dt,
                                float *const *dL_dc_k, float *const *dL_dt_k, hipStream_t stream);

/* Workspace bytes gs_compact_grads needs for n Gaussians. */
size_t gs_compact_workspace_bytes(int64_t n);

/* Zero-gradient elision (ByteSplat section 3 Insight 4, section 6): keeps the Gaussians
 * whose 9 screen-space gradient fields are not all exactly zero (-0.0 counts as zero)
 * and writes records {uint32 index_base + i, float g[9]} (40 bytes each) in ascending
 * index order to `records` (capacity n records), sets bit i%32 of bitmap[i/32] for each
 * kept Gaussian (bitmap [ceil(n/32)]), and reads the record count back to the host
 * (*r_out, host; synchronises `stream`). */
gs_status gs_compact_grads(const float *grads2d, int64_t n, uint32_t index_base, void *records,
                           uint32_t *bitmap, int64_t *r_out, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* One renderer partition's compacted records, as gs_compact_grads wrote them, and the
 * forward-communication index that maps its positions to the owner's Gaussians. */
typedef struct {
    const void *records;          /* r records {uint32 index; float g[9]} (40 B), 4-byte aligned */
    int64_t r;                    /* record count (the r_out of gs_compact_grads) */
    uint32_t index_base;          /* the index_base the records were written with */
    const uint32_t *owner_index;  /* [n_part]: owner Gaussian of partition position i; NULL: i itself */
    int64_t n_part;               /* positions in the partition */
} gs_grad_records;

/* Owner-side sparse decoding (ByteSplat section 6.2, Fig. 9): for every record of the k
 * partitions (0 <= k <= 16), position i = index - index_base is mapped through
 * owner_index to the owner Gaussian o and each non-zero field f is added to
 * grads2d[f * n_owner + o] with an fp32 atomic add.  grads2d ([9][n_owner], same field
 * order as gs_raster_bwd) is accumulated, not cleared; records of different partitions
 * that name the same Gaussian are summed in an unspecified order.  A record whose
 * position is outside [0, n_part) or whose owner Gaussian is outside [0, n_owner) is
 * skipped and counted into *rejected (device uint32, accumulated; may be NULL).  The
 * records and owner_index arrays are device memory, `parts` is a host array.  Calls
 * whose partitions are decoded into the same grads2d may overlap on different streams. */
gs_status gs_decode_grads(const gs_grad_records *parts, int32_t k, float *grads2d, int64_t n_owner,
                          uint32_t *rejected, hipStream_t stream);

/* The owner's update from screen-space gradients already summed per Gaussian (grads2d
 * [9][n], same field order as gs_raster_bwd; e.g. rebuilt by gs_decode_grads, ByteSplat
 * section 6.2): per Gaussian in one pass, the projection backward of gs_project_bwd, the
 * Adam update of gs_adam_step with those 3D gradients (which are never stored) and, if
 * next_cam is non-NULL, the projection of the updated Gaussian for next_cam into next_proj
 * (as gs_project(g, next_cam, p, next_proj) would write it afterwards; Splaxel section 2
 * "Projection").  The result equals gs_project_bwd, gs_adam_step and gs_project in
 * sequence, bit for bit.  grads2d is read only.  m, v, lr, step, beta1, beta2, eps: as
 * gs_grad_aggregate_adam.  Errors as gs_project_bwd, gs_adam_step and gs_project. */
gs_status gs_project_bwd_adam(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                              const float *grads2d, const gs_param_grads *m, const gs_param_grads *v,
                              const gs_adam_lrs *lr, int32_t step, float beta1, float beta2, float eps,
                              const gs_camera *next_cam, gs_projected *next_proj, hipStream_t stream);

/* Message describing the last non-OK status returned on the calling thread. */
const char *gs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
