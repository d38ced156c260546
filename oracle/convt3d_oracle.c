/*
 * convt3d_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for ConvTranspose3d (NCDHW,
 * cubic kernel, any stride / padding / output_padding) and the three
 * epilogues that follow it on the pages:
 *   - ReLU then GroupNorm            (p61 page, its statement of GroupNorm:
 *                                     per (sample, group) mean and biased
 *                                     variance, eps inside the square root,
 *                                     per-channel affine);
 *   - softmax over channels, sigmoid (p49 page, its max-subtracted softmax
 *                                     followed by 1/(1+exp(-v)));
 *   - x scale, training-mode BatchNorm3d, global average pool
 *                                    (p77 page, its statement of batch
 *                                     statistics over (N, D, H, W) with the
 *                                     biased variance, then the mean over
 *                                     D, H, W), with the running-statistics
 *                                     update of a training step, and the
 *                                     evaluation-mode variant that uses the
 *                                     running statistics.
 *
 * Every sum is accumulated in double precision; float inputs are widened on
 * read.  Only tests, the package smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The GPU library shares no code with it.
 *
 * Parity status: every function here is pinned by the CPU tests (library
 * routines for the same operation, the pages' worked examples, the stride-1
 * and adjoint identities, closed-form spatial sums and the normalisation
 * invariants); none is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Output length of a transposed convolution along one dimension:
 * (in - 1) * stride - 2 * pad + k + out_pad  (p49 page and p77 page, where the
 * output size of ConvTranspose3d is worked out before anything else). */
long oracle_out_dim(long in, long k, long s, long p, long op)
{
    return (in - 1) * s - 2 * p + k + op;
}

/*
 * Scatter definition of the transposed convolution (p49 page, where each
 * input voxel (d_in, h_in, w_in) and kernel tap (kd, kh, kw) add
 * weight * input to the output voxel d_in*s - p + kd (and likewise for h, w);
 * targets outside the output are dropped).  Weight layout [Cin, Cout, k, k, k]
 * as nn.ConvTranspose3d stores it.  y is [N, Cout, Do, Ho, Wo] and starts at
 * the bias (or 0 when b is NULL).
 *
 * The loops visit every (input channel, tap, input voxel) triple of an output
 * channel exactly once; the order in which a sum is taken is free.  Work is
 * split over (n, co): each thread owns whole output channels.
 */
void oracle_convt3d(const float *x, const float *w, const float *b,
                    int N, int Cin, int Cout, int D, int H, int W,
                    int k, int s, int p, int op, double *y)
{
    const long Do = oracle_out_dim(D, k, s, p, op);
    const long Ho = oracle_out_dim(H, k, s, p, op);
    const long Wo = oracle_out_dim(W, k, s, p, op);
    if (Do <= 0 || Ho <= 0 || Wo <= 0) return;
    const long S = Do * Ho * Wo;
    const long Sin = (long)D * H * W;
    const long kk = (long)k * k * k;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < N; ++n) {
        for (int co = 0; co < Cout; ++co) {
            double *yc = y + ((size_t)n * Cout + co) * (size_t)S;
            const double init = b ? (double)b[co] : 0.0;
            for (long i = 0; i < S; ++i) yc[i] = init;
            for (int ci = 0; ci < Cin; ++ci) {
                const float *xc = x + ((size_t)n * Cin + ci) * (size_t)Sin;
                const float *wc = w + ((size_t)ci * Cout + co) * (size_t)kk;
                for (int kd = 0; kd < k; ++kd)
                for (int kh = 0; kh < k; ++kh)
                for (int kw = 0; kw < k; ++kw) {
                    const double wv = (double)wc[((long)kd * k + kh) * k + kw];
                    for (int id = 0; id < D; ++id) {
                        const long od = (long)s * id - p + kd;
                        if (od < 0 || od >= Do) continue;
                        for (int ih = 0; ih < H; ++ih) {
                            const long oh = (long)s * ih - p + kh;
                            if (oh < 0 || oh >= Ho) continue;
                            const float *xrow = xc + ((long)id * H + ih) * W;
                            double *yrow = yc + (od * Ho + oh) * Wo;
                            for (int iw = 0; iw < W; ++iw) {
                                const long ow = (long)s * iw - p + kw;
                                if (ow < 0 || ow >= Wo) continue;
                                yrow[ow] += (double)xrow[iw] * wv;
                            }
                        }
                    }
                }
            }
        }
    }
}

/*
 * The same scatter definition for the general nn.ConvTranspose3d geometry:
 * per-dimension kernel size k[], stride s[], padding p[], output padding op[]
 * and dilation dl[] (index 0 = D, 1 = H, 2 = W), and `groups` channel groups.
 * Tap t along a dimension sits dl*t from the first one, so input i reaches
 * output s*i - p + dl*t; the output length is (in - 1)*s - 2p + dl*(k - 1) +
 * op + 1.  With groups G, output channel co belongs to group g = co / (Cout/G)
 * and sums only over input channels g*(Cin/G) .. (g+1)*(Cin/G) - 1; the weight
 * is [Cin, Cout/G, kD, kH, kW] (nn.ConvTranspose3d's layout).  The pages fix
 * groups = 1 and dilation = 1 and a cubic kernel; this is the module's own
 * definition for the other values.
 */
long oracle_out_dim_general(long in, long k, long s, long p, long op, long dl)
{
    return (in - 1) * s - 2 * p + dl * (k - 1) + op + 1;
}

void oracle_convt3d_general(const float *x, const float *w, const float *b,
                            int N, int Cin, int Cout, int D, int H, int W,
                            const int *k, const int *s, const int *p, const int *op,
                            const int *dl, int groups, double *y)
{
    const long Do = oracle_out_dim_general(D, k[0], s[0], p[0], op[0], dl[0]);
    const long Ho = oracle_out_dim_general(H, k[1], s[1], p[1], op[1], dl[1]);
    const long Wo = oracle_out_dim_general(W, k[2], s[2], p[2], op[2], dl[2]);
    if (Do <= 0 || Ho <= 0 || Wo <= 0 || groups < 1 || Cin % groups || Cout % groups) return;
    const long S = Do * Ho * Wo;
    const long Sin = (long)D * H * W;
    const long kk = (long)k[0] * k[1] * k[2];
    const int cig = Cin / groups, cog = Cout / groups;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < N; ++n) {
        for (int co = 0; co < Cout; ++co) {
            double *yc = y + ((size_t)n * Cout + co) * (size_t)S;
            const double init = b ? (double)b[co] : 0.0;
            for (long i = 0; i < S; ++i) yc[i] = init;
            const int g = co / cog, col = co % cog;
            for (int cl = 0; cl < cig; ++cl) {
                const int ci = g * cig + cl;
                const float *xc = x + ((size_t)n * Cin + ci) * (size_t)Sin;
                const float *wc = w + ((size_t)ci * cog + col) * (size_t)kk;
                for (int kd = 0; kd < k[0]; ++kd)
                for (int kh = 0; kh < k[1]; ++kh)
                for (int kw = 0; kw < k[2]; ++kw) {
                    const double wv = (double)wc[((long)kd * k[1] + kh) * k[2] + kw];
                    for (int id = 0; id < D; ++id) {
                        const long od = (long)s[0] * id - p[0] + (long)dl[0] * kd;
                        if (od < 0 || od >= Do) continue;
                        for (int ih = 0; ih < H; ++ih) {
                            const long oh = (long)s[1] * ih - p[1] + (long)dl[1] * kh;
                            if (oh < 0 || oh >= Ho) continue;
                            const float *xrow = xc + ((long)id * H + ih) * W;
                            double *yrow = yc + (od * Ho + oh) * Wo;
                            for (int iw = 0; iw < W; ++iw) {
                                const long ow = (long)s[2] * iw - p[2] + (long)dl[2] * kw;
                                if (ow < 0 || ow >= Wo) continue;
                                yrow[ow] += (double)xrow[iw] * wv;
                            }
                        }
                    }
                }
            }
        }
    }
}

/* Does tap kk of an output index o come from an input index?  Gather form of
 * the same relation (p49 page): o receives tap kk iff (o + p - kk) is a
 * non-negative multiple of s, from i = (o + p - kk) / s, if i < in. */
static int gather_index(long o, long kk, long s, long p, long in, long *i_out)
{
    const long t = o + p - kk;
    if (t < 0 || t % s != 0) return 0;
    const long i = t / s;
    if (i >= in) return 0;
    *i_out = i;
    return 1;
}

/* One output value by the gather form: the bias plus, for every input channel
 * and every tap whose source index is an in-range input voxel, x * w. */
double oracle_convt3d_point(const float *x, const float *w, const float *b,
                            int N, int Cin, int Cout, int D, int H, int W,
                            int k, int s, int p, int op,
                            int n, int co, long od, long oh, long ow)
{
    (void)N; (void)op;
    const long Sin = (long)D * H * W;
    const long kk = (long)k * k * k;
    double acc = b ? (double)b[co] : 0.0;
    for (int ci = 0; ci < Cin; ++ci) {
        const float *xc = x + ((size_t)n * Cin + ci) * (size_t)Sin;
        const float *wc = w + ((size_t)ci * Cout + co) * (size_t)kk;
        for (int kd = 0; kd < k; ++kd) {
            long id;
            if (!gather_index(od, kd, s, p, D, &id)) continue;
            for (int kh = 0; kh < k; ++kh) {
                long ih;
                if (!gather_index(oh, kh, s, p, H, &ih)) continue;
                for (int kw = 0; kw < k; ++kw) {
                    long iw;
                    if (!gather_index(ow, kw, s, p, W, &iw)) continue;
                    acc += (double)xc[(id * H + ih) * W + iw] *
                           (double)wc[((long)kd * k + kh) * k + kw];
                }
            }
        }
    }
    return acc;
}

/* The whole output by the gather form (small inputs only; a cross-check of
 * the scatter form). */
void oracle_convt3d_gather(const float *x, const float *w, const float *b,
                           int N, int Cin, int Cout, int D, int H, int W,
                           int k, int s, int p, int op, double *y)
{
    const long Do = oracle_out_dim(D, k, s, p, op);
    const long Ho = oracle_out_dim(H, k, s, p, op);
    const long Wo = oracle_out_dim(W, k, s, p, op);
    if (Do <= 0 || Ho <= 0 || Wo <= 0) return;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Cout; ++co)
            for (long od = 0; od < Do; ++od)
                for (long oh = 0; oh < Ho; ++oh)
                    for (long ow = 0; ow < Wo; ++ow)
                        y[((((size_t)n * Cout + co) * Do + od) * Ho + oh) * Wo + ow] =
                            oracle_convt3d_point(x, w, b, N, Cin, Cout, D, H, W, k, s, p, op,
                                                 n, co, od, oh, ow);
}

/*
 * ReLU then GroupNorm (p61 page): r = max(y, 0); for every (n, g) over the
 * channels [g*C/G, (g+1)*C/G) and all S positions, mean = sum(r)/cnt and the
 * biased variance var = sum((r - mean)^2)/cnt (two passes); then
 * out = (r - mean) / sqrt(var + eps) * gamma[c] + beta[c].
 * gamma/beta may be NULL (no affine).  stats, when not NULL, receives
 * [N, G, 2] = (mean, 1/sqrt(var + eps)).
 */
void oracle_relu_groupnorm(const double *y, int N, int C, long S, int G, double eps,
                           const float *gamma, const float *beta,
                           double *out, double *stats)
{
    const int cpg = C / G;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            const size_t base = ((size_t)n * C + (size_t)g * cpg) * (size_t)S;
            const double cnt = (double)cpg * (double)S;
            double sum = 0.0;
            for (size_t i = 0; i < (size_t)cpg * S; ++i) {
                const double r = y[base + i] > 0.0 ? y[base + i] : 0.0;
                sum += r;
            }
            const double mean = sum / cnt;
            double ss = 0.0;
            for (size_t i = 0; i < (size_t)cpg * S; ++i) {
                const double r = y[base + i] > 0.0 ? y[base + i] : 0.0;
                ss += (r - mean) * (r - mean);
            }
            const double var = ss / cnt;
            const double rstd = 1.0 / sqrt(var + eps);
            if (stats) {
                stats[((size_t)n * G + g) * 2 + 0] = mean;
                stats[((size_t)n * G + g) * 2 + 1] = rstd;
            }
            for (int cc = 0; cc < cpg; ++cc) {
                const int c = g * cpg + cc;
                const double ga = gamma ? (double)gamma[c] : 1.0;
                const double be = beta ? (double)beta[c] : 0.0;
                for (long i = 0; i < S; ++i) {
                    const size_t j = base + (size_t)cc * S + i;
                    const double r = y[j] > 0.0 ? y[j] : 0.0;
                    out[j] = (r - mean) * rstd * ga + be;
                }
            }
        }
    }
}

/*
 * Softmax over the channel dimension, then sigmoid (p49 page): per (n, voxel),
 * m = max_c y, e_c = exp(y_c - m), p_c = e_c / sum_j e_j,
 * out_c = 1 / (1 + exp(-p_c)).  The channel stride of NCDHW is S.
 * p, when not NULL, receives the softmax values themselves.
 */
void oracle_softmax_sigmoid(const double *y, int N, int C, long S, double *out, double *p)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n) {
        for (long v = 0; v < S; ++v) {
            const double *yv = y + (size_t)n * C * S + v;
            double m = yv[0];
            for (int c = 1; c < C; ++c)
                if (yv[(size_t)c * S] > m) m = yv[(size_t)c * S];
            double sum = 0.0;
            for (int c = 0; c < C; ++c) sum += exp(yv[(size_t)c * S] - m);
            for (int c = 0; c < C; ++c) {
                const size_t j = (size_t)n * C * S + (size_t)c * S + v;
                const double pc = exp(y[j] - m) / sum;
                if (p) p[j] = pc;
                out[j] = 1.0 / (1.0 + exp(-pc));
            }
        }
    }
}

/*
 * x scale, training-mode BatchNorm3d, AdaptiveAvgPool3d(1) (p77 page):
 * z = scale * y; per channel c, over all (n, d, h, w): mean_c and the biased
 * variance var_c (two passes); bn = (z - mean_c) / sqrt(var_c + eps) *
 * gamma[c] + beta[c]; out[n, c] = mean over (d, h, w) of bn.
 * stats, when not NULL, receives [C, 2] = (mean_c, var_c) of z.
 */
void oracle_scale_bn_avgpool(const double *y, int N, int C, long S, double scale, double eps,
                             const float *gamma, const float *beta,
                             double *out, double *stats)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int c = 0; c < C; ++c) {
        const double cnt = (double)N * (double)S;
        double sum = 0.0;
        for (int n = 0; n < N; ++n) {
            const double *yc = y + ((size_t)n * C + c) * (size_t)S;
            for (long i = 0; i < S; ++i) sum += scale * yc[i];
        }
        const double mean = sum / cnt;
        double ss = 0.0;
        for (int n = 0; n < N; ++n) {
            const double *yc = y + ((size_t)n * C + c) * (size_t)S;
            for (long i = 0; i < S; ++i) {
                const double d = scale * yc[i] - mean;
                ss += d * d;
            }
        }
        const double var = ss / cnt;
        const double rstd = 1.0 / sqrt(var + eps);
        const double ga = gamma ? (double)gamma[c] : 1.0;
        const double be = beta ? (double)beta[c] : 0.0;
        if (stats) {
            stats[(size_t)c * 2 + 0] = mean;
            stats[(size_t)c * 2 + 1] = var;
        }
        for (int n = 0; n < N; ++n) {
            const double *yc = y + ((size_t)n * C + c) * (size_t)S;
            double acc = 0.0;
            for (long i = 0; i < S; ++i)
                acc += (scale * yc[i] - mean) * rstd * ga + be;
            out[(size_t)n * C + c] = acc / (double)S;
        }
    }
}

/*
 * BatchNorm running statistics after one training step (p77 page: in training
 * mode BatchNorm3d normalises with the batch statistics and moves its running
 * mean and variance toward them by the momentum, 0.1 there).  The variance
 * folded in is the unbiased one, var * count / (count - 1), as nn.BatchNorm3d
 * keeps it (the pages name that module; they fix the biased estimator only for
 * the normalisation itself):
 *   rmean = (1 - momentum) * rmean + momentum * mean_c
 *   rvar  = (1 - momentum) * rvar  + momentum * var_c * count / (count - 1)
 * stats is [C, 2] = (batch mean, biased batch variance); count = N*D*H*W > 1.
 */
void oracle_bn_running_update(const double *stats, int C, double count, double momentum,
                              double *rmean, double *rvar)
{
    for (int c = 0; c < C; ++c) {
        const double mean = stats[(size_t)c * 2 + 0];
        const double unbiased = stats[(size_t)c * 2 + 1] * count / (count - 1.0);
        rmean[c] = (1.0 - momentum) * rmean[c] + momentum * mean;
        rvar[c] = (1.0 - momentum) * rvar[c] + momentum * unbiased;
    }
}

/*
 * x scale, BatchNorm3d in evaluation mode, AdaptiveAvgPool3d(1) (p77 page,
 * where the model in eval mode normalises with its running mean and variance
 * instead of batch statistics): z = scale * y;
 * bn = (z - rmean[c]) / sqrt(rvar[c] + eps) * gamma[c] + beta[c];
 * out[n, c] = mean over (d, h, w) of bn.  Every element is normalised and
 * then averaged, as written; no shortcut through the spatial sum.
 * gamma/beta NULL mean 1/0; rmean/rvar NULL mean 0/1 (a fresh module).
 */
void oracle_scale_bn_eval_avgpool(const double *y, int N, int C, long S, double scale, double eps,
                                  const float *gamma, const float *beta,
                                  const float *rmean, const float *rvar, double *out)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int c = 0; c < C; ++c) {
            const double ga = gamma ? (double)gamma[c] : 1.0;
            const double be = beta ? (double)beta[c] : 0.0;
            const double rm = rmean ? (double)rmean[c] : 0.0;
            const double rv = rvar ? (double)rvar[c] : 1.0;
            const double *yc = y + ((size_t)n * C + c) * (size_t)S;
            double acc = 0.0;
            for (long i = 0; i < S; ++i)
                acc += (scale * yc[i] - rm) / sqrt(rv + eps) * ga + be;
            out[(size_t)n * C + c] = acc / (double)S;
        }
    }
}

/* Number of OpenMP threads the library would use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
