// HIP kernels of libconvt3d for gfx950 around the convolution kernel: the
// statistics and normalisation passes of the fused epilogues, the standalone
// epilogue passes over a conv output the caller holds, and the evaluation-mode
// BatchNorm + pool path, which needs no convolution.
//
//  * gn_finalize_kernel   -- per (n, group) fp64 merge of statistics partials
//                            (sums around per-channel pivots), mean / biased
//                            variance / rstd, per-channel a, b.
//  * normalize_kernel     -- out = a[n,c] * v + b[n,c] with v = src (or
//                            ReLU(src)), float4, in place when src == out.
//  * bn_finalize_kernel   -- per channel fp64 batch mean / biased variance,
//                            the pooled output and the running statistics.
//  * row_stats_kernel     -- per (n, c, chunk) sums of v and v^2 over a conv
//                            output held in memory (v = ReLU(y) or scale*y).
//  * softmax_rows_kernel  -- channel softmax then sigmoid over a conv output in
//                            memory, one read and one write: the channels of a
//                            position in the registers of one or more waves
//                            (up to 1024 channels); softmax_pass_kernel, for
//                            more, reads twice (running max and sum of
//                            exponentials, then the result).
//  * bn_eval_rows_kernel  -- eval-mode BatchNorm + pool from per-row sums.
//  * eval_pack_kernel     -- tap-summed weights per input bin (eval mode).
//  * eval_binsum_kernel   -- sums of x over the input bins of each (n, cin).
//  * eval_finalize_kernel -- pooled conv mean = bias + bin sums . weights / S,
//                            then BatchNorm with the running statistics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "conv_index.hpp"
#include "convt3d_internal.hpp"

namespace convt3d {

namespace {

constexpr int kNormUnroll = 4;        // loads in flight per thread in the HBM passes
// Statistics merges: one workgroup per (n, group) or per channel reads all of
// its partial sums.  Few workgroups, so each needs many bytes in flight:
// 1024 threads with 8 partial-sum pairs in flight each.
constexpr int kStatThreads = 1024;
constexpr int kStatUnroll = 8;
constexpr int64_t kStreamBytes = int64_t(512) << 20;  // above this a pass streams past the 256 MB cache
constexpr float kLog2e = 1.4426950408889634f;

// exp(x) as 2^(x log2 e) on the hardware exp2 (relative error a few ulp).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Sum of two values over a 256-thread workgroup, same order every run.
// red holds 4 float2; every thread gets the result.
__device__ __forceinline__ float2 block_sum2(float a, float b, float2 *red) {
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off);
        b += __shfl_xor(b, off);
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(a, b);
    __syncthreads();
    const float2 r = make_float2((red[0].x + red[1].x) + (red[2].x + red[3].x),
                                 (red[0].y + red[1].y) + (red[2].y + red[3].y));
    __syncthreads();  // red may be reused
    return r;
}

// Sum of two doubles over a kStatThreads workgroup in a fixed order: a 64-lane
// xor-shuffle tree per wave, then the wave totals in wave order.  red holds
// kStatThreads / 64 double2; every thread gets the result.
__device__ __forceinline__ double2 block_sum2_f64(double a, double b, double2 *red) {
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off);
        b += __shfl_xor(b, off);
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_double2(a, b);
    __syncthreads();
    double2 r = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) {
        r.x += red[w].x;
        r.y += red[w].y;
    }
    __syncthreads();  // red may be reused
    return r;
}

template <class V>
__device__ __forceinline__ float *comps(V &v) { return reinterpret_cast<float *>(&v); }
template <class V>
constexpr int ncomp() { return (int)(sizeof(V) / sizeof(float)); }

}  // namespace

// ---------------------------------------------------------------------------
// Pivot of the statistics partials of (n, c): the partial sums are of
// v - pivot.  prow (one per (n, c) row, written by the statistics pass over y)
// takes precedence; else from the conv bias: relu(bias) for GroupNorm, scale *
// bias for BatchNorm; else 0.
__device__ __forceinline__ double stat_pivot(const float *prow, const float *pbias, bool relu, float scale, int n,
                                             int C, int c) {
    if (prow) return (double)prow[(size_t)n * C + c];
    if (!pbias) return 0.0;
    return relu ? (double)fmaxf(pbias[c], 0.0f) : (double)scale * (double)pbias[c];
}

// GroupNorm statistics: one workgroup per (n, group); fp64 sums of the fp32
// partials (layout [n][C][tile][2], sums of v - pivot(n, c)) in a fixed order,
// the pivots added back (sum v = sum d + cnt*p, sum v^2 = sum (d^2 + 2 p d) +
// cnt*p^2 per summed channel), then mean, biased variance E[v^2] - mean^2 (in
// fp64: the pivots keep the fp32 sums free of the mean's magnitude), rstd =
// 1/sqrt(var + eps), and per channel a = gamma*rstd, b = beta - mean*a.
// chan_step: every chan_step-th channel holds a sum (of chan_step channels
// around that channel's pivot).
__global__ __launch_bounds__(kStatThreads) void gn_finalize_kernel(const float *partials, int tiles_per_n, int C,
                                                          int G, int chan_step, float eps, const float *gamma,
                                                          const float *beta, float *ab, float *stats_out,
                                                          double count, const float *prow, const float *pbias,
                                                          double chan_count) {
    const int n = blockIdx.x / G, g = blockIdx.x % G;
    const int cpg = C / G;
    const int cps = cpg / chan_step;  // channels of the group that hold sums
    const int items = tiles_per_n * cps;
    double a1 = 0.0, a2 = 0.0;
    for (int i0 = threadIdx.x; i0 < items; i0 += blockDim.x * kStatUnroll) {
        float2 v[kStatUnroll];
        double pv[kStatUnroll];
#pragma unroll
        for (int u = 0; u < kStatUnroll; ++u) {
            const int i = i0 + u * (int)blockDim.x;
            v[u] = make_float2(0.0f, 0.0f);
            pv[u] = 0.0;
            if (i < items) {
                // tile fastest: each summed channel's tiles are contiguous
                const int k = i / tiles_per_n, t = i - k * tiles_per_n, cc = k * chan_step;
                v[u] = *reinterpret_cast<const float2 *>(partials +
                                                          ix::partial_offset(n, C, g * cpg + cc, tiles_per_n, t));
                pv[u] = stat_pivot(prow, pbias, true, 1.0f, n, C, g * cpg + cc);
            }
        }
#pragma unroll
        for (int u = 0; u < kStatUnroll; ++u) {
            a1 += (double)v[u].x;
            a2 += (double)v[u].y + 2.0 * pv[u] * (double)v[u].x;
        }
    }
    __shared__ double2 red[kStatThreads / 64];
    __shared__ double mean_s, rstd_s;
    const double2 tot = block_sum2_f64(a1, a2, red);
    if (threadIdx.x == 0) {
        double s1 = tot.x, s2 = tot.y;
        for (int cc = 0; cc < cpg; cc += chan_step) {  // each summed channel's pivot, over its values
            const double p = stat_pivot(prow, pbias, true, 1.0f, n, C, g * cpg + cc);
            s1 += chan_count * p;
            s2 += chan_count * p * p;
        }
        const double mean = s1 / count;
        double var = s2 / count - mean * mean;
        if (var < 0.0) var = 0.0;
        mean_s = mean;
        rstd_s = 1.0 / sqrt(var + (double)eps);
        if (stats_out) {
            stats_out[((size_t)n * G + g) * 2 + 0] = (float)mean;
            stats_out[((size_t)n * G + g) * 2 + 1] = (float)rstd_s;
        }
    }
    __syncthreads();
    for (int cc = threadIdx.x; cc < cpg; cc += blockDim.x) {
        const int c = g * cpg + cc;
        const double ga = gamma ? (double)gamma[c] : 1.0;
        const double be = beta ? (double)beta[c] : 0.0;
        const double a = ga * rstd_s;
        ab[((size_t)n * C + c) * 2 + 0] = (float)a;
        ab[((size_t)n * C + c) * 2 + 1] = (float)(be - mean_s * a);
    }
}

// Streaming load / store that bypasses cache retention (NT), or plain ones.
template <bool NT, class V>
__device__ __forceinline__ V load_stream(const V *p) {
    if constexpr (NT && sizeof(V) == 16) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
        return *reinterpret_cast<const V *>(&t);
    } else if constexpr (NT) {
        const float t = __builtin_nontemporal_load(reinterpret_cast<const float *>(p));
        return *reinterpret_cast<const V *>(&t);
    } else {
        return *p;
    }
}
template <bool NT, class V>
__device__ __forceinline__ void store_stream(V *p, const V &v) {
    if constexpr (NT && sizeof(V) == 16) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(*reinterpret_cast<const f4 *>(&v), reinterpret_cast<f4 *>(p));
    } else if constexpr (NT) {
        __builtin_nontemporal_store(*reinterpret_cast<const float *>(&v), reinterpret_cast<float *>(p));
    } else {
        *p = v;
    }
}

// GroupNorm normalisation, out = a[n,c] * v + b[n,c] with v = src or
// ReLU(src).  Block row y is one (n, c) channel (rows beyond gridDim.y are
// taken in further passes), so (a, b) is one scalar load; each thread issues
// kNormUnroll loads before its stores to keep enough bytes in flight for HBM.
// src == out is the in-place form.  NT: non-temporal loads, for tensors well
// past the 256 MB last-level cache (a tensor the conv has just written and
// that still partly sits in that cache reads faster without); NTS:
// non-temporal stores.
template <class V, bool RELU, bool NT, bool NTS>
__global__ __launch_bounds__(256) void normalize_kernel(const V *src, V *out, const float2 *ab, int rows,
                                                        int row_len) {
    for (int row = blockIdx.y; row < rows; row += gridDim.y) {
        const float2 p = ab[row];
        const V *s = src + (size_t)row * row_len;
        V *o = out + (size_t)row * row_len;
        const int base = blockIdx.x * (256 * kNormUnroll) + threadIdx.x;
        V v[kNormUnroll];
#pragma unroll
        for (int k = 0; k < kNormUnroll; ++k) {
            const int i = base + k * 256;
            if (i < row_len) v[k] = load_stream<NT>(s + i);
        }
#pragma unroll
        for (int k = 0; k < kNormUnroll; ++k) {
            const int i = base + k * 256;
            if (i < row_len) {
                float *c = comps(v[k]);
#pragma unroll
                for (int e = 0; e < ncomp<V>(); ++e) {
                    const float x = RELU ? fmaxf(c[e], 0.0f) : c[e];
                    c[e] = fmaf(p.x, x, p.y);
                }
                store_stream<NTS>(o + i, v[k]);
            }
        }
    }
}

// BatchNorm (training) + average pool: one workgroup per channel.  partials
// is [n][C][tile][2] of sums of z - pivot(n, c) and their squares, z = scale
// * y (the pivot added back in fp64 as in the GroupNorm merge).  Writes the
// pooled [n, C] output, the batch statistics and, when both buffers are
// given, the running statistics (unbiased variance folded in).
__global__ __launch_bounds__(kStatThreads) void bn_finalize_kernel(const float *partials, int N, int tiles_per_n, int C,
                                                          double S, float eps, const float *gamma,
                                                          const float *beta, float *out, float *stats_out,
                                                          float momentum, float *rmean, float *rvar,
                                                          const float *prow, const float *pbias, float pscale) {
    const int c = blockIdx.x;
    double a1 = 0.0, a2 = 0.0;
    const int items = N * tiles_per_n;
    // a per-sample pivot (from the statistics pass over y) enters each item's
    // cross term 2*p*sum; a per-channel one (from the bias) is added once below
    const double pc = prow ? 0.0 : stat_pivot(nullptr, pbias, false, pscale, 0, C, c);
    for (int i0 = threadIdx.x; i0 < items; i0 += blockDim.x * kStatUnroll) {
        float2 v[kStatUnroll];
        double pv[kStatUnroll];
#pragma unroll
        for (int u = 0; u < kStatUnroll; ++u) {
            const int i = i0 + u * (int)blockDim.x;  // i = n*tiles_per_n + t
            const int n = i / tiles_per_n, t = i - n * tiles_per_n;
            v[u] = i < items ? *reinterpret_cast<const float2 *>(partials + ix::partial_offset(n, C, c, tiles_per_n, t))
                             : make_float2(0.0f, 0.0f);
            pv[u] = prow && i < items ? (double)prow[(size_t)n * C + c] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kStatUnroll; ++u) {
            a1 += (double)v[u].x;
            a2 += (double)v[u].y + 2.0 * pv[u] * (double)v[u].x;
        }
    }
    __shared__ double2 red[kStatThreads / 64];
    __shared__ double mean_s, rstd_s;
    const double2 tot = block_sum2_f64(a1, a2, red);
    if (threadIdx.x == 0) {
        double s1 = tot.x, s2 = tot.y + 2.0 * pc * tot.x;
        for (int n = 0; n < N; ++n) {  // each sample's pivot, over its S values
            const double p = stat_pivot(prow, pbias, false, pscale, n, C, c);
            s1 += S * p;
            s2 += S * p * p;
        }
        const double cnt = (double)N * S;
        const double mean = s1 / cnt;
        double var = s2 / cnt - mean * mean;
        if (var < 0.0) var = 0.0;
        mean_s = mean;
        rstd_s = 1.0 / sqrt(var + (double)eps);
        if (stats_out) {
            stats_out[(size_t)c * 2 + 0] = (float)mean;
            stats_out[(size_t)c * 2 + 1] = (float)var;
        }
        if (rmean && rvar) {  // cnt > 1 is checked on the host
            const double m = (double)momentum;
            rmean[c] = (float)((1.0 - m) * (double)rmean[c] + m * mean);
            rvar[c] = (float)((1.0 - m) * (double)rvar[c] + m * var * cnt / (cnt - 1.0));
        }
    }
    __syncthreads();
    const double ga = gamma ? (double)gamma[c] : 1.0;
    const double be = beta ? (double)beta[c] : 0.0;
    // pooled output: one wave per sample sums that sample's tile partials
    // (lane l takes tiles l, l + 64, ...; then a fixed xor-shuffle tree)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int n0 = 0; n0 < N; n0 += (int)blockDim.x >> 6) {
        const int n = n0 + wave;  // uniform within the wave
        double m = 0.0;
        if (n < N)
            for (int t = lane; t < tiles_per_n; t += 64)
                m += (double)partials[ix::partial_offset(n, C, c, tiles_per_n, t)];
        for (int off = 32; off > 0; off >>= 1) m += __shfl_xor(m, off);
        if (n < N && lane == 0) {
            const double zbar = m / S + stat_pivot(prow, pbias, false, pscale, n, C, c);
            out[(size_t)n * C + c] = (float)((zbar - mean_s) * rstd_s * ga + be);
        }
    }
}

// ---------------------------------------------------------------------------
// Statistics of a conv output in memory: workgroup (chunk, row) sums
// d = v - p over elements [chunk*chunk_len, (chunk+1)*chunk_len) of row =
// n*C + c, with v = ReLU(mult*y) (RELU) or mult*y and the row's pivot p = v
// of the row's first element (every workgroup of the row reads it; the first
// chunk's writes it to pivots[row]); writes (sum d, sum d^2) to
// partials[n][C][chunk][2], the layout the finalize kernels read.  The pivot
// is a value of the row, so a large common offset does not cancel in the fp32
// sum of squares.
template <class V, bool RELU>
__global__ __launch_bounds__(256) void row_stats_kernel(const V *y, int rows, int row_len, int chunk_len,
                                                        int chunks, int C, float mult, float *partials,
                                                        float *pivots) {
    __shared__ float2 red[4];
    for (int row = blockIdx.y; row < rows; row += gridDim.y) {
        const V *p = y + (size_t)row * row_len;
        float pv = mult * reinterpret_cast<const float *>(p)[0];
        if (RELU) pv = fmaxf(pv, 0.0f);
        const int beg = blockIdx.x * chunk_len;
        const int end = min(row_len, beg + chunk_len);
        float s1 = 0.0f, s2 = 0.0f;
        for (int i0 = beg + (int)threadIdx.x; i0 < end; i0 += 256 * kNormUnroll) {
            V v[kNormUnroll];
#pragma unroll
            for (int k = 0; k < kNormUnroll; ++k)
                if (i0 + k * 256 < end) v[k] = p[i0 + k * 256];
#pragma unroll
            for (int k = 0; k < kNormUnroll; ++k)
                if (i0 + k * 256 < end) {
                    const float *c = comps(v[k]);
#pragma unroll
                    for (int e = 0; e < ncomp<V>(); ++e) {
                        float a = mult * c[e];
                        if (RELU) a = fmaxf(a, 0.0f);
                        a -= pv;
                        s1 += a;
                        s2 = fmaf(a, a, s2);
                    }
                }
        }
        const float2 r = block_sum2(s1, s2, red);
        if (threadIdx.x == 0) {
            const int n = row / C, c = row - n * C;
            float *pp = partials + ix::partial_offset(n, C, c, chunks, blockIdx.x);
            pp[0] = r.x;
            pp[1] = r.y;
            if (blockIdx.x == 0) pivots[row] = pv;
        }
    }
}

// Channel softmax then sigmoid of a conv output in memory, [n][C][S] with S
// counted in V units.  Thread = (n, one V of positions).  Pass 1 keeps a
// running max m and sum l of exp(v - m) over the channels, four channels per
// rescale; pass 2 reads the channels again and writes 1/(1 + exp(-p)) with
// p = exp(v - m) / l.  out may equal src.
template <class V, bool NT>
__global__ __launch_bounds__(256) void softmax_pass_kernel(const V *src, V *out, int N, int C, int S) {
    const int s = blockIdx.x * 256 + threadIdx.x;
    if (s >= S) return;
    constexpr int NC = ncomp<V>();
    for (int n = blockIdx.y; n < N; n += gridDim.y) {
        const V *p = src + (size_t)n * C * S + s;
        V *o = out + (size_t)n * C * S + s;
        float m[NC], l[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            m[e] = -INFINITY;
            l[e] = 0.0f;
        }
        int c = 0;
        for (; c + 4 <= C; c += 4) {
            V v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = load_stream<NT>(p + (size_t)(c + j) * S);
#pragma unroll
            for (int e = 0; e < NC; ++e) {
                const float a0 = comps(v[0])[e], a1 = comps(v[1])[e], a2 = comps(v[2])[e], a3 = comps(v[3])[e];
                const float mn = fmaxf(m[e], fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)));
                l[e] = l[e] * fast_exp(m[e] - mn) +
                       ((fast_exp(a0 - mn) + fast_exp(a1 - mn)) + (fast_exp(a2 - mn) + fast_exp(a3 - mn)));
                m[e] = mn;
            }
        }
        for (; c < C; ++c) {
            V v = load_stream<NT>(p + (size_t)c * S);
#pragma unroll
            for (int e = 0; e < NC; ++e) {
                const float a = comps(v)[e];
                const float mn = fmaxf(m[e], a);
                l[e] = l[e] * fast_exp(m[e] - mn) + fast_exp(a - mn);
                m[e] = mn;
            }
        }
        float inv[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) inv[e] = __builtin_amdgcn_rcpf(l[e]);
        for (c = 0; c < C; ++c) {
            V v = load_stream<NT>(p + (size_t)c * S);
            float *a = comps(v);
#pragma unroll
            for (int e = 0; e < NC; ++e) {
                const float pr = fast_exp(a[e] - m[e]) * inv[e];
                a[e] = __builtin_amdgcn_rcpf(1.0f + fast_exp(-pr));
            }
            store_stream<NT>(o + (size_t)c * S, v);
        }
    }
}

// Channel softmax then sigmoid of a conv output in memory, [n][C][S], with
// one read and one write.  A position group is WPP waves (WPP = ceil(C / CR))
// covering 64*VEC positions: lane l of the group's wave w holds channels
// [w*CR, (w+1)*CR) of positions s0 + VEC*l .. + VEC-1 in registers, so every
// channel row of the group is one coalesced access of 256*VEC bytes.  The
// waves combine their maxima and sums of exponentials through LDS in a fixed
// order.  A workgroup holds blockDim / (64*WPP) position groups.  sigmoid of
// the probability q = e/sum is 1/2 + q R(q^2), R the polynomial of
// kSigmoidOdd, evaluated in e^2 with coefficients scaled by powers of 1/sum.  out may equal src (each thread
// writes only what it read).  NT: non-temporal loads (tensors past the
// last-level cache); the output, which nothing here reads again, is stored
// non-temporally.  S is counted in VEC-vectors.
template <int CR, int VEC, bool NT>
__global__ __launch_bounds__(1024) void softmax_rows_kernel(const float *src, float *out, int N, int C, int S,
                                                            int WPP) {
    typedef float vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ float red[1024 * VEC];  // [wave][lane][VEC]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = wave / WPP, wq = wave - grp * WPP;
    const int groups = (int)blockDim.x / (64 * WPP);
    const int s = (blockIdx.x * groups + grp) * 64 + lane;  // in vectors
    const bool live = s < S;
    const int c0 = wq * CR;
    const int nc = min(CR, C - c0);                          // channels of this wave (the last may hold fewer)
    const int gw0 = (grp * WPP * 64 + lane) * VEC;           // LDS slot of this lane in the group's first wave
    for (int n = blockIdx.y; n < N; n += gridDim.y) {
        const vec_t *p = reinterpret_cast<const vec_t *>(src) + ((size_t)n * C + c0) * S + s;
        vec_t v[CR];
#pragma unroll
        for (int c = 0; c < CR; ++c) {
            v[c] = -INFINITY;
            if (live && c < nc) {
                if constexpr (NT) v[c] = __builtin_nontemporal_load(p + (size_t)c * S);
                else v[c] = p[(size_t)c * S];
            }
        }
        float m[VEC], l[VEC], d[VEC][4];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            m[e] = v[0][e];
#pragma unroll
            for (int c = 1; c < CR; ++c) m[e] = fmaxf(m[e], v[c][e]);
        }
        if (WPP > 1) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) red[threadIdx.x * VEC + e] = m[e];
            __syncthreads();
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                m[e] = red[gw0 + e];
                for (int j = 1; j < WPP; ++j) m[e] = fmaxf(m[e], red[gw0 + 64 * VEC * j + e]);
            }
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float ml = m[e] * kLog2e;
            l[e] = 0.0f;
#pragma unroll
            for (int c = 0; c < CR; ++c) {
                v[c][e] = __builtin_amdgcn_exp2f(fmaf(v[c][e], kLog2e, -ml));  // 0 for unused (-inf) entries
                l[e] += v[c][e];
            }
        }
        if (WPP > 1) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) red[threadIdx.x * VEC + e] = l[e];
            __syncthreads();
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                l[e] = red[gw0 + e];
                for (int j = 1; j < WPP; ++j) l[e] += red[gw0 + 64 * VEC * j + e];
            }
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float inv = __builtin_amdgcn_rcpf(l[e]);
            const float inv2 = inv * inv;
            float ik = inv;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                d[e][k] = kSigmoidOdd[k] * ik;
                ik *= inv2;
            }
        }
        vec_t *o = reinterpret_cast<vec_t *>(out) + ((size_t)n * C + c0) * S + s;
#pragma unroll
        for (int c = 0; c < CR; ++c) {
            if (!live || c >= nc) continue;
            vec_t y;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float x = v[c][e], x2 = x * x;
                float t = d[e][3];
#pragma unroll
                for (int k = 2; k >= 0; --k) t = fmaf(t, x2, d[e][k]);
                y[e] = fmaf(t, x, 0.5f);
            }
            __builtin_nontemporal_store(y, o + (size_t)c * S);
        }
    }
}

// Eval-mode BatchNorm + pool from per-row sums (partials [n][C][chunk][2] of
// (sum (y - pivot), -), pivots [n][C]): thread per (n, c), pooled mean
// m = scale * (sum / S + pivot), then
// out = (scale*m - rmean) / sqrt(rvar + eps) * gamma + beta.
__global__ __launch_bounds__(256) void bn_eval_rows_kernel(const float *partials, int N, int chunks, int C,
                                                           double S, float scale, float eps, const float *gamma,
                                                           const float *beta, const float *rmean,
                                                           const float *rvar, float *out, const float *pivots) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= N * C) return;
    const int n = i / C, c = i - n * C;
    double sum = 0.0;
    for (int t = 0; t < chunks; ++t) sum += (double)partials[ix::partial_offset(n, C, c, chunks, t)];
    const double m = (double)scale * (sum / S + (double)pivots[i]);
    const double ga = gamma ? (double)gamma[c] : 1.0, be = beta ? (double)beta[c] : 0.0;
    const double mu = rmean ? (double)rmean[c] : 0.0, var = rvar ? (double)rvar[c] : 1.0;
    out[i] = (float)((m - mu) / sqrt(var + (double)eps) * ga + be);
}

// ---------------------------------------------------------------------------
// Evaluation-mode BatchNorm + pool without the convolution.  Along each dim
// the input range splits into bins [cut[j], cut[j+1]); tap t reaches the
// output from exactly the inputs [lo[t], hi1[t]), a union of whole bins.  So
//   sum_o y[n,co,o] = S*bias[co] + sum_ci sum_bins R[n,ci,bin] * Wb[co,ci,bin]
// with R the sum of x over the bin box and Wb the sum of w over the taps whose
// input range holds the bin.

__device__ __forceinline__ int bin_of(const EvalGeom &E, int b, int dim) {
    if (dim == 0) return b / (E.nb[1] * E.nb[2]);
    if (dim == 1) return (b / E.nb[2]) % E.nb[1];
    return b % E.nb[2];
}

// Wb[co][ci_local][bin] (ci_local: input channel within co's group): one
// wave per weight row [ci][co_local] of kD*kH*kW taps.  The workgroup first
// turns the bin tables into one bit mask per (dim, tap) in LDS: bit j set when
// bin j of that dim lies in the tap's input range.
__global__ __launch_bounds__(256) void eval_pack_kernel(const EvalGeom E, const float *w, float *wb) {
    __shared__ unsigned long long mask[3][kEvalMaxK];
    for (int i = threadIdx.x; i < 3 * kEvalMaxK; i += blockDim.x) {
        const int d = i / kEvalMaxK, t = i - d * kEvalMaxK;
        unsigned long long m = 0;
        if (t < E.k3[d])
            for (int j = 0; j < E.nb[d]; ++j)
                if (E.lo[d][t] <= E.cut[d][j] && E.cut[d][j + 1] <= E.hi1[d][t]) m |= 1ull << j;
        mask[d][t] = m;
    }
    __syncthreads();
    const int pair = blockIdx.x * 4 + (int)(threadIdx.x >> 6);  // ci*cog + co_local
    const int lane = threadIdx.x & 63;
    if (pair >= E.Cin * E.cog) return;
    const int ci = pair / E.cog, col = pair - ci * E.cog;
    const int grp = ci / E.cig, cil = ci - grp * E.cig, co = grp * E.cog + col;
    const int kh_ = E.k3[1], kw_ = E.k3[2], khw = kh_ * kw_, kk = E.k3[0] * khw;
    const float *row = w + (size_t)pair * kk;
    for (int b = 0; b < E.nbins; ++b) {
        const int bd = bin_of(E, b, 0), bh = bin_of(E, b, 1), bw = bin_of(E, b, 2);
        double acc = 0.0;
        for (int t = lane; t < kk; t += 64) {
            const int td = t / khw, th = (t / kw_) % kh_, tw = t % kw_;
            if ((mask[0][td] >> bd) & (mask[1][th] >> bh) & (mask[2][tw] >> bw) & 1ull) acc += (double)row[t];
        }
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) wb[((size_t)co * E.cig + cil) * E.nbins + b] = (float)acc;
    }
}

// Sum of x over the box [da,db) x [ha,hb) x [wa,wb) of one plane, this
// wave's share (4 waves).  Rows are dealt to lanes so that a row of up to 64
// vectors (VEC: float4, else float) is one coalesced wave access, and each
// lane issues 4 row loads before it adds; wider rows loop over the lanes.
template <bool VEC>
__device__ float box_sum(const float *xp, int H, int W, int da, int db, int ha, int hb, int wa, int wb,
                         int lane, int wave) {
    constexpr int U = 4;
    const int bh_len = hb - ha;
    const int nrows = (db - da) * bh_len;
    const int width = VEC ? (wb - wa) >> 2 : (wb - wa);
    auto load = [&](const float *rowp, int i) {
        if (VEC) {
            const float4 v = reinterpret_cast<const float4 *>(rowp)[i];
            return (v.x + v.y) + (v.z + v.w);
        }
        return rowp[i];
    };
    // row r of the box -> (dd, hh), advanced by `step` rows at a time
    float acc = 0.0f;
    if (width <= 64) {
        const int rpi = 64 / width;            // rows per wave access
        const int lr = lane / width, lw = lane - lr * width;
        if (lr >= rpi) return 0.0f;
        const int step = 4 * rpi;              // rows per workgroup step
        const int sd = step / bh_len, sh = step - sd * bh_len;
        int r = wave * rpi + lr;
        int dd = r / bh_len, hh = r - dd * bh_len;
        for (; r < nrows; r += U * step) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                v[u] = 0.0f;
                if (r + u * step < nrows) v[u] = load(xp + ((size_t)(da + dd) * H + (ha + hh)) * W + wa, lw);
                dd += sd;
                hh += sh;
                if (hh >= bh_len) {
                    hh -= bh_len;
                    ++dd;
                }
            }
            acc += (v[0] + v[1]) + (v[2] + v[3]);
        }
    } else {
        int dd = wave / bh_len, hh = wave - (wave / bh_len) * bh_len;
        const int sd = 4 / bh_len, sh = 4 - sd * bh_len;
        for (int r = wave; r < nrows; r += 4) {
            const float *rowp = xp + ((size_t)(da + dd) * H + (ha + hh)) * W + wa;
            int i = lane;
            for (; i + (U - 1) * 64 < width; i += U * 64) {
                float v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load(rowp, i + u * 64);
                acc += (v[0] + v[1]) + (v[2] + v[3]);
            }
            for (; i < width; i += 64) acc += load(rowp, i);
            dd += sd;
            hh += sh;
            if (hh >= bh_len) {
                hh -= bh_len;
                ++dd;
            }
        }
    }
    return acc;
}

// R[plane][chunk][bin]: workgroup = (plane = n*Cin + ci, d-chunk).
__global__ __launch_bounds__(256) void eval_binsum_kernel(const EvalGeom E, const float *x, float *R) {
    const int plane = blockIdx.x / E.nchunk, chunk = blockIdx.x - plane * E.nchunk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d0 = chunk * E.dchunk, d1 = min(E.D, d0 + E.dchunk);
    const float *xp = x + (size_t)plane * E.D * E.H * E.W;
    float *Rp = R + ((size_t)plane * E.nchunk + chunk) * E.nbins;
    __shared__ float red[4];
    for (int b = 0; b < E.nbins; ++b) {
        const int bd = bin_of(E, b, 0), bh = bin_of(E, b, 1), bw = bin_of(E, b, 2);
        const int da = max(E.cut[0][bd], d0), db = min(E.cut[0][bd + 1], d1);
        const int ha = E.cut[1][bh], hb = E.cut[1][bh + 1], wa = E.cut[2][bw], wb = E.cut[2][bw + 1];
        float acc = 0.0f;
        if (da < db) {
            if (((wa | wb | E.W) & 3) == 0) acc = box_sum<true>(xp, E.H, E.W, da, db, ha, hb, wa, wb, lane, wave);
            else acc = box_sum<false>(xp, E.H, E.W, da, db, ha, hb, wa, wb, lane, wave);
        }
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) red[wave] = acc;
        __syncthreads();
        if (threadIdx.x == 0) Rp[b] = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
    }
}

// out[n, co]: one wave per (n, co); fp64 dot product of the chunk-summed bin
// sums with Wb, then BatchNorm with the running statistics.
__global__ __launch_bounds__(256) void eval_finalize_kernel(const EvalGeom E, const float *R, const float *wb,
                                                            const float *bias, float scale, float eps,
                                                            const float *gamma, const float *beta,
                                                            const float *rmean, const float *rvar, float *out) {
    const int item = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= E.N * E.Cout) return;
    const int n = item / E.Cout, co = item - n * E.Cout;
    const int K = E.cig * E.nbins;           // input channels of co's group x bins
    const int ci0 = (co / E.cog) * E.cig;
    double acc = 0.0;
    for (int j = lane; j < K; j += 64) {
        const int ci = ci0 + j / E.nbins, b = j % E.nbins;
        const float *r = R + ((size_t)(n * E.Cin + ci) * E.nchunk) * E.nbins + b;
        double rs = 0.0;
        for (int c = 0; c < E.nchunk; ++c) rs += (double)r[(size_t)c * E.nbins];
        acc += rs * (double)wb[(size_t)co * K + j];
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
        const double m = (bias ? (double)bias[co] : 0.0) + acc * E.inv_S;
        const double ga = gamma ? (double)gamma[co] : 1.0, be = beta ? (double)beta[co] : 0.0;
        const double mu = rmean ? (double)rmean[co] : 0.0, var = rvar ? (double)rvar[co] : 1.0;
        out[item] = (float)(((double)scale * m - mu) / sqrt(var + (double)eps) * ga + be);
    }
}

// ---------------------------------------------------------------------------
// launchers

// Threads of a statistics merge over `items` partial-sum pairs: enough waves
// for kStatUnroll pairs in flight per thread, up to kStatThreads.  A short
// merge (the standalone passes' few chunks per row) runs as one wave, which
// finishes sooner than a full workgroup of idle threads.
static int stat_threads(int64_t items) {
    const int64_t waves = (items + 64 * kStatUnroll - 1) / (64 * kStatUnroll);
    return (int)std::min<int64_t>(kStatThreads, std::max<int64_t>(1, waves) * 64);
}

int launch_gn_finalize(const float *partials, int N, int tiles_per_n, int C, int G, int chan_step, double count,
                       float eps, const float *gamma, const float *beta, float *ab, float *stats_out,
                       const float *prow, const float *pbias, double S, void *stream) {
    const int threads = stat_threads((int64_t)tiles_per_n * (C / G / chan_step));
    hipLaunchKernelGGL(gn_finalize_kernel, dim3(N * G), dim3(threads), 0, (hipStream_t)stream, partials,
                       tiles_per_n, C, G, chan_step, eps, gamma, beta, ab, stats_out, count, prow, pbias,
                       (double)chan_step * S);
    return (int)hipGetLastError();
}

template <class V, bool RELU, bool NT, bool NTS>
static void launch_normalize_t(const float *src, float *out, const float *ab, int rows, int len, void *stream) {
    const int gx = (len + 256 * kNormUnroll - 1) / (256 * kNormUnroll);
    const int gy = rows < 65535 ? rows : 65535;
    hipLaunchKernelGGL((normalize_kernel<V, RELU, NT, NTS>), dim3(gx, gy), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const V *>(src), reinterpret_cast<V *>(out),
                       reinterpret_cast<const float2 *>(ab), rows, len);
}

template <class V, bool RELU>
static void launch_normalize_nt(const float *src, float *out, const float *ab, int rows, int len, bool nt,
                                bool nts, void *stream) {
    if (nt && nts) launch_normalize_t<V, RELU, true, true>(src, out, ab, rows, len, stream);
    else if (nt) launch_normalize_t<V, RELU, true, false>(src, out, ab, rows, len, stream);
    else if (nts) launch_normalize_t<V, RELU, false, true>(src, out, ab, rows, len, stream);
    else launch_normalize_t<V, RELU, false, false>(src, out, ab, rows, len, stream);
}

// stream_out: the output is not read again soon (a standalone epilogue's
// result): store it non-temporally whatever its size
int launch_normalize(const float *src, float *out, const float *ab, int rows, int64_t S, bool relu,
                     void *stream, bool stream_out) {
    const bool vec = S % 4 == 0;
    const int len = (int)(vec ? S / 4 : S);
    // measured: non-temporal access pays for a 1.07 GB tensor (+5 %) and
    // costs for a 0.32 GB one just written by the conv (-4 %)
    const bool nt = (double)rows * (double)S * sizeof(float) > (double)kStreamBytes;
    const bool nts = nt || stream_out;
    if (vec) {
        if (relu) launch_normalize_nt<float4, true>(src, out, ab, rows, len, nt, nts, stream);
        else launch_normalize_nt<float4, false>(src, out, ab, rows, len, nt, nts, stream);
    } else {
        if (relu) launch_normalize_nt<float, true>(src, out, ab, rows, len, nt, nts, stream);
        else launch_normalize_nt<float, false>(src, out, ab, rows, len, nt, nts, stream);
    }
    return (int)hipGetLastError();
}

int launch_bn_finalize(const float *partials, int N, int tiles_per_n, int C, double S, const convt3d_epilogue &e,
                       float *out, const float *prow, const float *pbias, void *stream) {
    // and at least one wave per sample for the pooled output's per-sample sums
    const int threads = std::max(stat_threads((int64_t)N * tiles_per_n), std::min(kStatThreads, 64 * N));
    hipLaunchKernelGGL(bn_finalize_kernel, dim3(C), dim3(threads), 0, (hipStream_t)stream, partials, N,
                       tiles_per_n, C, S, e.eps, e.gamma, e.beta, out, e.stats_out, e.momentum, e.running_mean,
                       e.running_var, prow, pbias, e.scale);
    return (int)hipGetLastError();
}

template <class V, bool RELU>
static void launch_row_stats_t(const float *y, int rows, int len, int chunks, int C, float mult, float *partials,
                               float *pivots, void *stream) {
    const int chunk_len = (len + chunks - 1) / chunks;
    const int gy = rows < 65535 ? rows : 65535;
    hipLaunchKernelGGL((row_stats_kernel<V, RELU>), dim3(chunks, gy), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const V *>(y), rows, len, chunk_len, chunks, C, mult, partials, pivots);
}

int launch_row_stats(const float *y, int N, int C, int64_t S, bool relu, float mult, float *partials,
                     float *pivots, void *stream) {
    const bool vec = S % 4 == 0;
    const int len = (int)(vec ? S / 4 : S);
    const int chunks = row_stat_chunks(S);
    const int rows = N * C;
    if (vec) {
        if (relu) launch_row_stats_t<float4, true>(y, rows, len, chunks, C, mult, partials, pivots, stream);
        else launch_row_stats_t<float4, false>(y, rows, len, chunks, C, mult, partials, pivots, stream);
    } else {
        if (relu) launch_row_stats_t<float, true>(y, rows, len, chunks, C, mult, partials, pivots, stream);
        else launch_row_stats_t<float, false>(y, rows, len, chunks, C, mult, partials, pivots, stream);
    }
    return (int)hipGetLastError();
}

int launch_softmax_pass(const float *src, float *out, int N, int C, int64_t S, void *stream) {
    const int gy = N < 65535 ? N : 65535;
    const bool nt = (double)N * C * (double)S * sizeof(float) > (double)kStreamBytes;
    if (C <= 1024) {  // every channel of a position in registers: one read of y
        // lanes hold CR channels x VEC positions (CR * VEC <= 64 registers);
        // measured on the 64- and 256-channel layers' y: two positions per lane
        // move 5.4 TB/s (the rate of a plain device copy), one 4.6-5.4, four 4.9-5.1
        int vec = 2;
        while (vec > 1 && (S % vec != 0 || C * vec > 1024)) vec /= 2;  // at most 16 waves per group
        const int cr_max = 64 / vec;
        const int CR = C <= cr_max / 4 ? cr_max / 4 : C <= cr_max / 2 ? cr_max / 2 : cr_max;
        const int wpp = (C + CR - 1) / CR;             // waves per position group (<= 16)
        {
            const int groups = wpp <= 4 ? 4 / wpp : 1;  // position groups per workgroup
            const int len = (int)(S / vec);
            const dim3 grid((len + 64 * groups - 1) / (64 * groups), gy), block(64 * wpp * groups);
            auto go = [&](auto kern) {
                hipLaunchKernelGGL(kern, grid, block, 0, (hipStream_t)stream, src, out, N, C, len, wpp);
            };
#define CONVT3D_SM(cr, v)                                                                        \
            if (CR == cr && vec == v) {                                                          \
                nt ? go(softmax_rows_kernel<cr, v, true>) : go(softmax_rows_kernel<cr, v, false>); \
                return (int)hipGetLastError();                                                   \
            }
            CONVT3D_SM(16, 1) CONVT3D_SM(32, 1) CONVT3D_SM(64, 1)
            CONVT3D_SM(8, 2) CONVT3D_SM(16, 2) CONVT3D_SM(32, 2)
            CONVT3D_SM(4, 4) CONVT3D_SM(8, 4) CONVT3D_SM(16, 4)
#undef CONVT3D_SM
            return (int)hipErrorInvalidValue;
        }
    }
    if (S % 4 == 0) {
        const int len = (int)(S / 4);
        const dim3 grid((len + 255) / 256, gy);
        const float4 *s4 = reinterpret_cast<const float4 *>(src);
        float4 *o4 = reinterpret_cast<float4 *>(out);
        if (nt)
            hipLaunchKernelGGL((softmax_pass_kernel<float4, true>), grid, dim3(256), 0, (hipStream_t)stream, s4, o4, N,
                               C, len);
        else
            hipLaunchKernelGGL((softmax_pass_kernel<float4, false>), grid, dim3(256), 0, (hipStream_t)stream, s4, o4,
                               N, C, len);
    } else {
        const int len = (int)S;
        const dim3 grid((len + 255) / 256, gy);
        if (nt)
            hipLaunchKernelGGL((softmax_pass_kernel<float, true>), grid, dim3(256), 0, (hipStream_t)stream, src, out,
                               N, C, len);
        else
            hipLaunchKernelGGL((softmax_pass_kernel<float, false>), grid, dim3(256), 0, (hipStream_t)stream, src, out,
                               N, C, len);
    }
    return (int)hipGetLastError();
}

int launch_bn_eval_rows(const float *partials, int N, int chunks, int C, double S, const convt3d_epilogue &e,
                        float *out, const float *pivots, void *stream) {
    const int items = N * C;
    hipLaunchKernelGGL(bn_eval_rows_kernel, dim3((items + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       partials, N, chunks, C, S, e.scale, e.eps, e.gamma, e.beta, e.running_mean, e.running_var,
                       out, pivots);
    return (int)hipGetLastError();
}

int launch_eval_pack(const EvalGeom &E, const float *w, float *wb, void *stream) {
    const int64_t pairs = (int64_t)E.Cin * E.cog;
    hipLaunchKernelGGL(eval_pack_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, (hipStream_t)stream, E,
                       w, wb);
    return (int)hipGetLastError();
}

int launch_eval_binsum(const EvalGeom &E, const float *x, float *R, void *stream) {
    const int64_t blocks = (int64_t)E.N * E.Cin * E.nchunk;
    hipLaunchKernelGGL(eval_binsum_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, E, x, R);
    return (int)hipGetLastError();
}

int launch_eval_finalize(const EvalGeom &E, const float *R, const float *wb, const float *bias,
                         const convt3d_epilogue &e, float *out, void *stream) {
    const int64_t items = (int64_t)E.N * E.Cout;
    hipLaunchKernelGGL(eval_finalize_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       E, R, wb, bias, e.scale, e.eps, e.gamma, e.beta, e.running_mean, e.running_var, out);
    return (int)hipGetLastError();
}

}  // namespace convt3d
