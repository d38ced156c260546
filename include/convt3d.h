/*
 * convt3d.h -- C ABI of libconvt3d: ConvTranspose3d (NCDHW, fp32) fused with
 * its epilogue, on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the three pages work on:
 *   y[n, co, o] = bias[co] + sum_ci sum_taps x[n, ci, i] * w[ci, co, tap]
 * over every (input voxel i, kernel tap) pair with o = stride*i - pad + tap in
 * each spatial dimension (p49 page, its scatter statement of the transposed
 * convolution; p77 page and p49 page, the output size
 * (in - 1)*stride - 2*pad + k + out_pad), and its general nn.ConvTranspose3d
 * form: per-dimension kernel size, stride, padding and output padding,
 * dilation dl (tap t sits dl*t from the first: o = stride*i - pad + dl*t,
 * output size (in - 1)*stride - 2*pad + dl*(k - 1) + out_pad + 1) and channel
 * groups (output channel co sums over the input channels of its group only);
 * the pages use groups 1, dilation 1 and cubic kernels.  Then one epilogue:
 *   - ReLU then GroupNorm (p61 page's statement of GroupNorm: per (n, group)
 *     mean and biased variance over channels of the group and all voxels, eps
 *     inside the square root, per-channel gamma/beta);
 *   - softmax over the channel dimension then sigmoid (p49 page: max-subtracted
 *     softmax, then 1/(1+exp(-v)));
 *   - multiply by `scale`, training-mode BatchNorm3d with batch statistics
 *     over (N, D, H, W) and the biased variance, then AdaptiveAvgPool3d(1)
 *     (p77 page); only the pooled [n, cout] result is produced.  The running
 *     statistics move toward the batch ones by the momentum (p77 page, its
 *     remark that training mode updates them), with the unbiased variance as
 *     nn.BatchNorm3d keeps it;
 *   - the same in evaluation mode (p77 page: the module in eval mode
 *     normalises with its running mean and variance): the pooled result is
 *     then an affine map of the spatial mean of y, which the p77 page reduces
 *     to input sums times tap-summed weights; no convolution is run.
 *
 * Conventions for every entry point:
 *   - All tensors are caller-owned, contiguous, fp32, in DEVICE memory of the
 *     current HIP device, 16-byte aligned.  The library never allocates or
 *     frees device memory and never synchronises the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every kernel is enqueued on it; results are ready in stream order.
 *   - A nonzero return is an error code (see convt3d_status_string); errors
 *     found from the arguments are returned before anything is launched and
 *     leave every output untouched.
 *   - Calls that share a workspace on overlapping streams race; give each
 *     concurrent call its own workspace.
 *   - The library links the HIP runtime by its soname (libamdhip64.so.7) and
 *     must share the runtime that owns the caller's memory and streams: load
 *     it after that runtime (with PyTorch, after importing torch, which
 *     carries its own copy).  Loaded first, it would pull in the system
 *     runtime and the caller's would be loaded beside it.
 */
#ifndef CONVT3D_H
#define CONVT3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Geometry.  Input x is [n, cin, d, h, w]; weight is [cin, cout/groups, k[0],
 * k[1], k[2]] (the layout nn.ConvTranspose3d stores).  Arrays are indexed
 * (0 = d, 1 = h, 2 = w).  Limits: n >= 0 (n == 0 is an empty batch: nothing is
 * launched), every other size >= 1, 1 <= stride <= 4, 0 <= pad,
 * 0 <= out_pad < max(stride, dilation) (nn.ConvTranspose3d's rule), groups
 * divides cin and cout, and each output dim >= 1. */
typedef struct convt3d_geom {
    int32_t n, cin, cout, d, h, w;
    int32_t k[3], stride[3], pad[3], out_pad[3], dilation[3];
    int32_t groups;
} convt3d_geom;

enum convt3d_epi_kind {
    CONVT3D_EPI_NONE = 0,                    /* out = y                                   */
    CONVT3D_EPI_RELU_GROUPNORM = 1,          /* out = GroupNorm(ReLU(y))                  */
    CONVT3D_EPI_SOFTMAX_SIGMOID = 2,         /* out = sigmoid(softmax_channels(y))        */
    CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL = 3,  /* out[n,c] = mean_dhw BN_train(scale * y)   */
    CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL = 4    /* out[n,c] = mean_dhw BN_eval(scale * y)    */
};

/* Epilogue description.
 *   kind      one of convt3d_epi_kind.
 *   groups    GroupNorm groups (cout % groups == 0); ignored otherwise.
 *   eps       GroupNorm / BatchNorm epsilon (added to the variance).
 *   scale     multiplier applied before BatchNorm; ignored otherwise.
 *   gamma     [cout] device, per-channel scale for GN/BN; NULL means 1.
 *   beta      [cout] device, per-channel shift for GN/BN; NULL means 0.
 *   stats_out optional device output, NULL to skip:
 *               GroupNorm: [n, groups, 2] = (mean, 1/sqrt(var + eps)) of ReLU(y);
 *               BatchNorm (training): [cout, 2] = (batch mean, biased batch
 *                                                  variance) of scale*y;
 *               others: ignored.
 *   momentum      BatchNorm training: weight of the batch statistics in the
 *                 running-statistics update (0.1 in nn.BatchNorm3d).
 *   running_mean  [cout] device.  BatchNorm training: when running_mean and
 *   running_var   running_var are both non-NULL they are updated in place,
 *                   rm = (1 - momentum) * rm + momentum * mean,
 *                   rv = (1 - momentum) * rv + momentum * var * M / (M - 1)
 *                 with M = n * Do * Ho * Wo values per channel (M > 1
 *                 required); both NULL: no update.  BatchNorm eval: read only;
 *                 NULL means 0 (mean) / 1 (variance), a fresh module.
 *                 Ignored by the other kinds. */
typedef struct convt3d_epilogue {
    int32_t kind;
    int32_t groups;
    float eps;
    float scale;
    const float *gamma;
    const float *beta;
    float *stats_out;
    float momentum;
    float *running_mean;
    float *running_var;
} convt3d_epilogue;

enum convt3d_status {
    CONVT3D_OK = 0,
    CONVT3D_ERR_NULL = 1,          /* a required pointer is NULL                      */
    CONVT3D_ERR_GEOMETRY = 2,      /* a size out of range or an empty output          */
    CONVT3D_ERR_GROUPS = 3,        /* GroupNorm groups < 1 or cout % groups != 0      */
    CONVT3D_ERR_ALIGNMENT = 4,     /* a tensor pointer is not 16-byte aligned         */
    CONVT3D_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than required         */
    CONVT3D_ERR_UNSUPPORTED = 6,   /* epilogue kind unknown or not valid for the call */
    CONVT3D_ERR_LAUNCH = 7,        /* HIP reported an error when launching            */
    CONVT3D_ERR_TOO_LARGE = 8,     /* a tensor exceeds 2^31 elements, or (conv path)  */
                                   /* an input channel plane D*H*W exceeds 2^29       */
    CONVT3D_ERR_ALIAS = 9,         /* out overlaps x                                  */
    CONVT3D_ERR_SCRATCH = 10       /* convt3d_fused_noalloc: the plan needs more workspace than the
                                      library's static scratch (CONVT3D_NOALLOC_SCRATCH_BYTES) */
};

/* Human-readable text for a status code (static storage). */
const char *convt3d_status_string(int status);

/* Output spatial size (Do, Ho, Wo) of the geometry.  Returns a status. */
int convt3d_output_dims(const convt3d_geom *geom, int32_t out_dhw[3]);

/* Number of fp32 elements `out` must hold: n*cout*Do*Ho*Wo for NONE / GN /
 * softmax, n*cout for the pooled BatchNorm epilogues; -1 on invalid input. */
int64_t convt3d_output_elems(const convt3d_geom *geom, const convt3d_epilogue *epi);

/* Bytes of the pre-packed weight buffer for this geometry (0 on invalid input). */
size_t convt3d_packed_weight_bytes(const convt3d_geom *geom);

/* Re-lay the nn.ConvTranspose3d weight w [cin, cout/groups, k...] (device) into
 * the per-group, per-stride-phase, matrix-core operand order the convolution
 * kernel reads (w_packed, device, convt3d_packed_weight_bytes bytes).  Enqueued
 * on stream; w_packed depends only on the geometry's channels, kernel size,
 * stride, pad, dilation and groups. */
int convt3d_prepack_weights(const convt3d_geom *geom, const float *w, void *w_packed,
                            void *stream);

/* The weight form of the evaluation-mode BatchNorm + pool epilogue, which runs
 * no convolution (p77 page, its reduction of the pooled output to input sums
 * times weights summed over the kernel taps).  Along each dimension the input
 * index range splits into at most 2k+1 bins, cut where some tap starts or
 * stops reaching the output; for every (cin, cout) pair and bin triple the
 * weights of the taps that reach the output from that whole bin are summed.
 * With pad 0 there is one bin (the whole input) and this is the tap sum.
 * Bytes of that buffer (0 on invalid input or a kernel size above 31): */
size_t convt3d_eval_weight_bytes(const convt3d_geom *geom);

/* Fill w_eval (device, convt3d_eval_weight_bytes bytes) from w [cin,
 * cout/groups, k...] (device).  Enqueued on stream.  convt3d_fused with the
 * kind CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL takes w_eval in place of w_packed. */
int convt3d_prepack_eval_weights(const convt3d_geom *geom, const float *w, void *w_eval,
                                 void *stream);

/* Bytes of device workspace convt3d_fused needs for (geom, epi) (statistics
 * partials and per-channel scale/shift), for every plan convt3d_autotune may
 * choose.  May be 0 (then workspace may be NULL). */
size_t convt3d_workspace_size(const convt3d_geom *geom, const convt3d_epilogue *epi);

/* The fused forward pass.
 *   x          [n, cin, d, h, w] device input.
 *   w_packed   output of convt3d_prepack_weights for this geometry (for
 *              CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL: of convt3d_prepack_eval_weights).
 *   bias       [cout] device, or NULL for no bias.
 *   out        device output, convt3d_output_elems(geom, epi) floats; must not
 *              overlap x.  For GroupNorm it is also used as the staging buffer
 *              of ReLU(y) before normalisation in place; for softmax with more
 *              than 128 channels or with groups > 1 (then one workgroup's tile
 *              does not hold every channel) it stages y, which a second pass
 *              turns into the result in place.
 * With groups > 1 one convolution launch covers every (sample, group) pair
 * (one launch per group when n * groups exceeds 65535).
 *   workspace  device scratch of at least convt3d_workspace_size bytes.
 * Enqueues 1 to 3 kernels on stream and returns without waiting. */
int convt3d_fused(const float *x, const void *w_packed, const float *bias,
                  const convt3d_geom *geom, const convt3d_epilogue *epi, float *out,
                  void *workspace, size_t workspace_bytes, void *stream);

/* The fused forward pass for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): convt3d_fused with the library's own static device scratch as
 * the workspace, so no workspace argument.  Same arguments otherwise, same
 * plan (the tuned one after convt3d_autotune), same kernels and results.
 * It allocates no device memory: the scratch is a device array of
 * CONVT3D_NOALLOC_SCRATCH_BYTES (32 MiB) that each device the library runs
 * on holds until the process ends; its address is looked up once per device
 * at that device's first call (the first call for a new geometry also plans
 * it on the host, as convt3d_fused does).  A plan needing more workspace than
 * the scratch returns CONVT3D_ERR_SCRATCH before anything is launched (use
 * convt3d_fused with a workspace of convt3d_workspace_size bytes instead).
 * Every call on one device shares that device's scratch: calls that overlap
 * on one device (different streams, or host threads) race.  Each call writes
 * every scratch word it reads before reading it, so the previous call's
 * contents are never cleared. */
#define CONVT3D_NOALLOC_SCRATCH_BYTES (32u << 20)
int convt3d_fused_noalloc(const float *x, const void *w_packed, const float *bias,
                          const convt3d_geom *geom, const convt3d_epilogue *epi, float *out,
                          void *stream);

/* Plan selection by timing.  The cost model ranks the kernel configurations
 * for (geom, epi); this runs the best few of them on the caller's buffers
 * (the same arguments as convt3d_fused; out and workspace are overwritten,
 * epi->stats_out too) and keeps the fastest for every later convt3d_fused
 * call with this geometry and epilogue kind in this process.  Every plan
 * computes the same result up to float summation order.  Unlike
 * convt3d_fused it waits on the device (it times the candidates with HIP
 * events on `stream`).  Candidates needing more workspace than
 * workspace_bytes are skipped.  BatchNorm running statistics are left
 * untouched (the timed calls do not update them).  result may be NULL.  The
 * best 12 configurations are timed, one plan each (environment
 * CONVT3D_TUNE_CANDIDATES=1..64 changes that; CONVT3D_TUNE_LOG prints one
 * line per candidate to stderr), then up to 8 other border segmentations of
 * the fastest one: after about 20 ms of warm-up calls, each in three rounds
 * of repeated calls (about 2 ms of work per round), its fastest round
 * counting. */
typedef struct convt3d_tune_result {
    int32_t candidates;      /* plans timed                                      */
    int32_t chosen;          /* rank of the chosen plan in cost-model order (0 = the model's pick;
                                ranks past the first list are the fastest configuration's other
                                border segmentations, timed in a second stage) */
    float chosen_ms;         /* time per call of the chosen plan                 */
    float model_choice_ms;   /* time per call of the cost model's pick           */
} convt3d_tune_result;

int convt3d_autotune(const float *x, const void *w_packed, const float *bias,
                     const convt3d_geom *geom, const convt3d_epilogue *epi, float *out,
                     void *workspace, size_t workspace_bytes, void *stream,
                     convt3d_tune_result *result);

/* The epilogue alone, on a conv output the caller already holds (for
 * instance from another convolution implementation): y is [n, c, spatial]
 * (NCDHW with the three spatial dims flattened, spatial = Do*Ho*Wo), device,
 * fp32.  Kinds: CONVT3D_EPI_RELU_GROUPNORM and CONVT3D_EPI_SOFTMAX_SIGMOID
 * write out [n, c, spatial] (out == y is allowed: in place; a partial overlap
 * is not); the two BatchNorm kinds write out [n, c] (must not overlap y), and
 * the training one updates the running statistics as convt3d_fused does (the
 * count M is n * spatial).  CONVT3D_EPI_NONE is rejected
 * (CONVT3D_ERR_UNSUPPORTED).  Same numerics as the fused epilogues; y is read
 * twice for GroupNorm (statistics, then the output pass), once for softmax
 * over up to 1024 channels (twice above that: running maximum and sum, then
 * the output) and once for BatchNorm.  Enqueued on stream, no waiting. */
size_t convt3d_epilogue_workspace_size(int32_t n, int32_t c, int64_t spatial, const convt3d_epilogue *epi);
int convt3d_epilogue_only(const float *y, int32_t n, int32_t c, int64_t spatial,
                          const convt3d_epilogue *epi, float *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Planner's choices for (geom, epi), for reporting and tests. */
typedef struct convt3d_plan_info {
    int32_t variant;           /* kernel variant id                                   */
    int32_t co_blocks_per_wave, pos_blocks_per_wave, w_phases_per_wave;
    int32_t waves_co, waves_pos; /* wave grid of one workgroup                       */
    int32_t tile_q[3];         /* box of stride-phase positions per workgroup (d,h,w) */
    int32_t ci_chunk;          /* input channels staged in LDS per step               */
    int32_t lds_bytes;         /* dynamic LDS per workgroup                           */
    int64_t workgroups;        /* conv kernel grid size                               */
    int64_t issued_macs;       /* multiply-adds the matrix cores execute (incl. padding) */
    int64_t valid_macs;        /* multiply-adds whose input voxel is in range          */
    int32_t phase_loop;        /* 1: a workgroup covers every (d, h) stride phase       */
    int32_t tuned;             /* 1: chosen by convt3d_autotune                         */
    int32_t border_split;      /* dims split into border / interior tile regions (bit 0 d, 1 h, 2 w);
                                  bit 3 + d (6 + d): only the low (high) border of dim d is a region
                                  of its own, the other border is tiled with the interior */
    int32_t xcd_order;         /* 0: phase / channel-tile index fastest per XCD, 1: tile fastest */
    int32_t softmax_pass;      /* 1: softmax runs as a second pass (cout > 128, groups) */
    int32_t eval_bins;         /* BN eval: input bins per (n, cin) plane, else 0        */
    int32_t conv_launches;     /* conv kernel launches per call: 1, or one per channel group
                                  when n * groups exceeds the grid's z limit (0: no conv) */
} convt3d_plan_info;

int convt3d_get_plan_info(const convt3d_geom *geom, const convt3d_epilogue *epi,
                          convt3d_plan_info *info);

/* Kernel timing for measurement.  Between convt3d_profile_begin() and
 * convt3d_profile_end(), every convt3d_fused call records HIP events on its
 * stream around each kernel it launches (convt3d_epilogue_only and the
 * pre-pack calls too).  convt3d_profile_end() waits for the
 * recorded events (it synchronises on them, so call it after the timed
 * region), fills `out` with the summed per-kernel durations and stops
 * recording.  Not thread-safe with respect to concurrent recording sessions. */
typedef struct convt3d_profile {
    int32_t calls;        /* convt3d_fused / convt3d_epilogue_only calls recorded */
    double conv_ms;       /* convolution (+ fused epilogue) kernel, summed        */
    double finalize_ms;   /* GroupNorm / BatchNorm statistics kernels, summed     */
    double normalize_ms;  /* output passes: GroupNorm normalisation, softmax      */
    double reduce_ms;     /* full-tensor sums: statistics of y, eval input bins   */
    double prepack_ms;    /* convt3d_prepack_weights / _eval_weights kernels      */
} convt3d_profile;

/* Kernel kinds convt3d_profile_begin_kinds records (bit mask); the fields of
 * convt3d_profile in the same order. */
#define CONVT3D_PROFILE_CONV 0x1u      /* conv_ms      */
#define CONVT3D_PROFILE_FINALIZE 0x2u  /* finalize_ms  */
#define CONVT3D_PROFILE_NORMALIZE 0x4u /* normalize_ms */
#define CONVT3D_PROFILE_REDUCE 0x8u    /* reduce_ms    */
#define CONVT3D_PROFILE_PREPACK 0x10u  /* prepack_ms   */
#define CONVT3D_PROFILE_ALL 0x1Fu

/* convt3d_profile_begin() records every kernel kind.  An event pair in the
 * stream costs a few microseconds per kernel, so a timed region that wants its
 * step time undisturbed records only the kind it needs:
 * convt3d_profile_begin_kinds(mask) records the kernels of the kinds in `mask`
 * (a nonzero subset of CONVT3D_PROFILE_ALL, else CONVT3D_ERR_UNSUPPORTED and
 * nothing changes); the fields of the other kinds stay 0. */
int convt3d_profile_begin(void);
int convt3d_profile_begin_kinds(uint32_t kinds);
int convt3d_profile_end(convt3d_profile *out);

#ifdef __cplusplus
}
#endif

#endif /* CONVT3D_H */
