// Internal declarations shared by the planner, the C-ABI and the kernels of
// libconvt3d.  Not part of the public interface (include/convt3d.h is).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "convt3d.h"

namespace convt3d {

constexpr int kMaxStride = 4;
constexpr int kMaxPhases = kMaxStride * kMaxStride * kMaxStride;
constexpr int kOctet = 8;          // input channels per packed weight group (4 MFMA k-steps)
constexpr int kMaxRegions = 27;    // tiling regions: (low border, interior, high border)^3
constexpr int kBlockThreads = 256; // 4 wavefronts per workgroup
constexpr int kMaxLdsBytes = 80 * 1024;  // at least two workgroups per CU
constexpr int kNumXcd = 8;               // MI355X: 8 XCDs (256 CUs), one L2 each
constexpr int64_t kL2Bytes = 4 << 20;    // L2 per XCD
constexpr int kRowStatChunk = 8192;      // vector elements per workgroup in the statistics pass over y
// Register-prefetch kernels hold the next chunk's halo (one octet) in
// registers: at most kRpPositions halo positions per thread.
constexpr int kRpPositions = 10;
// The conv kernel's halo staging addresses a chunk of CI_T input channel
// planes with 32-bit byte offsets when CI_T * D*H*W is at most
// kMaxChunkPlanes, else one channel plane per descriptor; input planes D*H*W
// stay at or below kMaxInputPlane.
constexpr int64_t kMaxChunkPlanes = int64_t(1) << 29;
constexpr int64_t kMaxInputPlane = int64_t(1) << 29;
constexpr int kEvalMaxK = 31;            // eval-mode BN: kernel size limit (bins per dim <= 2k+1)
constexpr int kEvalMaxBins = 2 * kEvalMaxK + 1;
constexpr int kEvalTargetBlocks = 2048;  // eval-mode bin sums: workgroups to aim for
// convt3d_autotune: kernel configurations timed (the cost model's best), then
// border segmentations of the fastest one; the workspace bound covers both
constexpr int kTuneCandidates = 12;
constexpr int kTuneBorderAlternatives = 8;

// sigmoid(p) for a softmax probability p in [0, 1]: sigmoid(p) - 1/2 is odd,
// approximated by p * (r0 + r1 p^2 + r2 p^4 + r3 p^6), the Chebyshev series of
// sigmoid - 1/2 on [-1, 1] truncated after T7, float32 (|error| < 1.2e-7 with
// Horner's rule in p^2; sigmoid_poly.py beside the kernels prints them).
constexpr float kSigmoidOdd[4] = {2.499994040e-01f, -2.082532272e-02f, 2.053756500e-03f, -1.693251979e-04f};

// Per-dimension stride-phase description.  Output index o = s*q + rho; the
// taps that reach it are t = r + ts*j (j = 0..J-1) from input i = q + c - e*j,
// where with dilation dl and g = gcd(dl, s): ts = s/g, e = dl/g, r is the
// smallest tap with dl*r = rho + pad (mod s) and c = (rho + pad - dl*r) / s.
// Without dilation: ts = s, e = 1, r = (rho + pad) mod s, c = (rho + pad) div s.
struct DimPhase {
    int r;   // first kernel tap of the phase
    int c;   // input offset of tap r (may be negative with dilation)
    int J;   // number of taps (0: no tap reaches this phase)
    int nq;  // number of q with s*q + rho < Out
};

// Arguments of the convolution kernel (passed by value).
struct ConvParams {
    const float *x;
    const float *wp;      // packed weights
    const float *bias;    // may be null
    float *out;
    float *partials;      // [n][cout][tiles_per_n][2] (channel-major) or null
    int N, Cin, Cout, D, H, W, Do, Ho, Wo;  // Cin, Cout: of one channel group
    int Cout_total;       // output channels of the whole conv (row stride of out and partials)
    int x_nstride;        // floats per sample of x (all groups' channels)
    int G;                // channel groups in this launch (grid z = sample * G + group); 1 when
                          // the host launches once per group with offset pointers
    int xg;               // floats from one group's first input channel to the next (cig * D*H*W)
    int wpg;              // floats from one group's packed weights to the next
    int s3[3];            // stride per dim
    int pe[3];            // input step per tap index j, per dim (dilation / gcd)
    int Qd, Qh, Qw;
    // Tiling regions.  rg[r] = {start d,h,w; end d,h,w; box d,h,w; tiles d,h,w}
    // in stride-phase coordinates q; workgroup x-index b belongs to region r when
    // rg_off[r] <= b < rg_off[r+1].
    int nreg;
    int rg[kMaxRegions][12];
    int rg_off[kMaxRegions + 1];
    int tiles_total;      // rg_off[nreg]
    int CI_T;             // input channels per LDS chunk (multiple of 8)
    int plane_desc;       // 1: CI_T * D*H*W > kMaxChunkPlanes, staging loads take one descriptor per plane
    int octets;           // ceil(Cin / 8)
    int nchunks;          // ceil(octets * 8 / CI_T)
    int cb_total;         // ceil(Cout / 32)
    int WCO, WPOS;        // wave grid
    int co_tiles;
    int nwgroups;         // w-phase groups per (rho_d, rho_h): s / NPH
    int order;            // 0: (co tile, phase) index fastest, 1: tile fastest
    int phase_loop;       // 1: each workgroup loops over all (rho_d, rho_h) groups
    int red_off;          // LDS float offset of the epilogue's reduction scratch
    int epi;
    int gn_block8;        // GroupNorm whose groups are whole 8-channel blocks: tile sums per block
    float scale;
    int tiles_per_n;
    int pr[3][kMaxStride], pc[3][kMaxStride], pJ[3][kMaxStride];
    int ntaps[kMaxPhases];
    int wp_off[kMaxPhases];   // float offset of each phase's packed block
    int steps4[kMaxPhases];   // packed float4 groups per co-block of each phase = octets*ntaps
};

// Evaluation-mode BatchNorm + pool (no convolution).  Along dim `dim` the
// input index range [0, in) splits into bins [cut[j], cut[j+1]), j < nb; tap t
// reaches the output from inputs [lo[t], hi1[t]) (lo >= hi1: from none), and
// every such range is a union of whole bins.
struct EvalGeom {
    int N, Cin, Cout, D, H, W;
    int cig, cog;                     // channels per group (input, output)
    int k3[3];
    int nb[3];
    int nbins;                        // nb[0] * nb[1] * nb[2]
    int cut[3][kEvalMaxBins + 1];
    int lo[3][kEvalMaxK], hi1[3][kEvalMaxK];
    int nchunk, dchunk;               // d-chunks per (n, cin) plane in the bin-sum kernel
    double inv_S;                     // 1 / (Do * Ho * Wo)
};

struct Plan {
    convt3d_geom g{};
    convt3d_epilogue e{};
    int Do = 0, Ho = 0, Wo = 0;
    int64_t S = 0;            // output voxels per channel
    int s3[3] = {1, 1, 1};    // stride per dim
    int ts[3] = {1, 1, 1};    // tap step per dim within a phase
    int pe[3] = {1, 1, 1};    // input step per dim per tap index
    int nph = 1;              // s3[0] * s3[1] * s3[2]
    int G = 1, cig = 1, cog = 1;  // channel groups, input / output channels per group
    int Q[3] = {0, 0, 0};     // ceil(Out / s)
    DimPhase ph[3][kMaxStride]{};
    int ntaps[kMaxPhases]{};
    int64_t wp_off[kMaxPhases]{};
    int steps4[kMaxPhases]{};
    int cb_total = 0, octets = 0;  // of one channel group
    int64_t packed_floats = 0;       // one group's packed weights (floats)
    // kernel choice
    int variant = -1;
    int CBW = 1, NPH = 1, PBW = 1, WCO = 1, WPOS = 1;
    int TQ[3] = {1, 1, 1};    // box of the largest region (for reporting)
    int nreg = 0;
    int rg[kMaxRegions][12]{};
    int rg_off[kMaxRegions + 1]{};
    int tiles_total = 0;
    int CI_T = 8, nchunks = 1;
    int lds_bytes = 0;
    int co_tiles = 1, nwgroups = 1;
    int phase_loop = 0, red_off = 0;
    int split = 0;            // dims split into border / interior segments (bit 0 d, 1 h, 2 w);
                              // bit 3 + d (6 + d): only the low (high) border of dim d on its own
    int softmax_pass = 0;     // softmax with cout > 128: conv stores y, a second pass finishes
    int eval = 0;             // eval-mode BatchNorm + pool: no conv (EvalGeom below)
    EvalGeom eg{};
    int order = 0;            // workgroup order within an XCD (see ConvParams::order)
    int64_t tiles_per_n = 0;
    int64_t grid_x = 0, grid_y = 0, grid_z = 0;
    int group_launch = 1;     // 1: one launch covers every channel group (grid z = n * G)
    int64_t issued_macs = 0, valid_macs = 0;
    // workspace layout (bytes)
    size_t ws_partials = 0, ws_ab = 0, ws_bins = 0, ws_bytes = 0;
};

// Kernel variants the library is built with.
struct Variant {
    int CBW, NPH, PBW;
    bool softmax;        // compiled with the softmax epilogue (else NONE / GN / BN)
    int waves_per_simd;  // register-limited occupancy of the compiled kernel
    bool phase_loop;     // also compiled with the (rho_d, rho_h) phase-group loop
    bool prefetch = false;  // register prefetch of the next channel chunk (one octet per chunk)
};
extern const Variant kVariants[];
extern const int kNumVariants;

int64_t out_dim(int64_t in, int64_t k, int64_t s, int64_t p, int64_t op, int64_t dl);
int validate_geom(const convt3d_geom *g);
int make_geometry(const convt3d_geom *g, Plan *pl);        // phases + packing only
int make_plan(const convt3d_geom *g, const convt3d_epilogue *e, Plan *pl);
// The max_k cheapest plans by the cost model, one per kernel configuration
// (variant, wave grid, box, chunk, phase loop); with `like`, only plans of that
// plan's configuration, one per border segmentation.
int plan_candidates(const convt3d_geom *g, const convt3d_epilogue *e, int max_k, std::vector<Plan> *out,
                    const Plan *like = nullptr);
void fill_conv_params(const Plan &pl, ConvParams *cp);
int make_eval_geom(const convt3d_geom *g, EvalGeom *eg);  // CONVT3D_ERR_UNSUPPORTED for k > kEvalMaxK
// Workspace bytes of the plan convt3d_fused runs for (g, e) now (api.cpp).
int current_plan_workspace(const convt3d_geom *g, const convt3d_epilogue *e, size_t *bytes);

// Launchers (kernels.hip: pre-pack and convolution).  Return a hipError_t as int.
// launch_prepack packs one channel group: w points at its [cig, cog, k...] slice.
int launch_prepack(const Plan &pl, const float *w, float *wp, void *stream);
int launch_conv(const Plan &pl, const ConvParams &cp, void *stream);

// Launchers (epilogue.hip).  partials are [n][chunk or tile][C][2]; the GroupNorm
// merge reads every chan_step-th channel (8 when the conv kept one sum per
// 8-channel block, at the block's first channel; else 1).
// Statistics partials are sums of v - pivot(n, c): the pivot is prow[n*C + c]
// when prow is given (the statistics pass over y writes it), else relu(bias)
// (GroupNorm) or scale*bias (BatchNorm) of pbias, else 0.
int launch_gn_finalize(const float *partials, int N, int tiles_per_n, int C, int G, int chan_step, double count,
                       float eps, const float *gamma, const float *beta, float *ab, float *stats_out,
                       const float *prow, const float *pbias, double S, void *stream);
int launch_normalize(const float *src, float *out, const float *ab, int rows, int64_t S, bool relu,
                     void *stream, bool stream_out = false);
int launch_bn_finalize(const float *partials, int N, int tiles_per_n, int C, double S, const convt3d_epilogue &e,
                       float *out, const float *prow, const float *pbias, void *stream);
int row_stat_chunks(int64_t S);
int launch_row_stats(const float *y, int N, int C, int64_t S, bool relu, float mult, float *partials,
                     float *pivots, void *stream);
int launch_softmax_pass(const float *src, float *out, int N, int C, int64_t S, void *stream);
int launch_bn_eval_rows(const float *partials, int N, int chunks, int C, double S, const convt3d_epilogue &e,
                        float *out, const float *pivots, void *stream);
int launch_eval_pack(const EvalGeom &E, const float *w, float *wb, void *stream);
int launch_eval_binsum(const EvalGeom &E, const float *x, float *R, void *stream);
int launch_eval_finalize(const EvalGeom &E, const float *R, const float *wb, const float *bias,
                         const convt3d_epilogue &e, float *out, void *stream);

}  // namespace convt3d
