// Host-side planner of libconvt3d: geometry checks, stride-phase tables,
// packed-weight layout, tile choice and workspace layout.
//
// Stride-phase split (p49 page, its gather relation: output o receives tap k
// iff (o + pad - k) is a multiple of the stride, from input (o + pad - k)/s).
// Writing o = s*q + rho, the taps that reach o are k = r + s*j with
// r = (rho + pad) mod s, from input i = q + c - j with c = (rho + pad) div s,
// j = 0 .. J-1, J = ceil((k - r)/s).  Each phase (rho_d, rho_h, rho_w) is a
// dense correlation over q with a J_d x J_h x J_w sub-kernel, so no tap that
// can never be valid is ever multiplied.  With dilation dl the taps sit dl
// apart: o receives tap t iff s divides (o + pad - dl*t); with g = gcd(dl, s)
// the taps of a phase are t = r + (s/g)*j and their inputs q + c - (dl/g)*j.
// Strides, kernel sizes, pads and dilations are per dimension; channel groups
// are independent convolutions run one after another.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "convt3d_internal.hpp"

namespace convt3d {

// Cost of one staging wait of a workgroup in MAC-equivalents (about 2000 CU
// cycles of idle MFMA at 128 MACs per cycle).
constexpr double kStageWaitMacs = 250e3;

// Kernel variants compiled into the library (co-blocks per wave, w-phases per
// wave, position blocks per wave).  Keep in sync with the instantiations in
// kernels.hip.
// waves_per_simd is the occupancy the compiled kernel's register count allows
// (used only by the cost model; the phase-loop build of a variant has the
// same occupancy as the plain one).
const Variant kVariants[] = {
    {1, 1, 8, false, 2, false}, {1, 1, 4, false, 4, true},  {1, 1, 2, false, 6, false},
    {1, 2, 4, false, 2, true},  {1, 2, 2, false, 4, true},
    {1, 1, 4, true, 4, false},  {1, 1, 2, true, 6, true},   {1, 2, 2, true, 4, true},
    {2, 1, 4, true, 2, false},  {2, 2, 2, true, 2, true},   {2, 1, 2, true, 3, true},
    {2, 2, 1, true, 3, true},
    {4, 1, 2, true, 1, false},  {4, 2, 1, true, 1, true},   {4, 1, 1, true, 3, true},
    // register prefetch of the next channel chunk, for layers whose halo (not
    // registers) holds the CU to two workgroups: a two-wave register budget
    {1, 1, 4, false, 2, false, true},
};
const int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int64_t out_dim(int64_t in, int64_t k, int64_t s, int64_t p, int64_t op, int64_t dl) {
    return (in - 1) * s - 2 * p + dl * (k - 1) + op + 1;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
// floor / ceil of a / b for b > 0 and any sign of a
static int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
static int64_t ceil_div_any(int64_t a, int64_t b) { return -floor_div(-a, b); }
static int gcd_int(int a, int b) { while (b) { const int t = a % b; a = b; b = t; } return a; }

// Tap index range [lo, hi] of a phase (input offset c, step e, J taps) that
// reaches the input [0, in) from some q of [q0, q0 + te - 1]: inputs are
// q + c - e*j.
static void live_taps(int q0, int te, int c, int e, int J, int in, int *lo, int *hi) {
    *lo = (int)std::max<int64_t>(0, ceil_div_any((int64_t)q0 + c - (in - 1), e));
    *hi = (int)std::min<int64_t>(J - 1, floor_div((int64_t)q0 + te - 1 + c, e));
}

int validate_geom(const convt3d_geom *g) {
    if (!g) return CONVT3D_ERR_NULL;
    if (g->n < 0 || g->cin < 1 || g->cout < 1 || g->d < 1 || g->h < 1 || g->w < 1 || g->groups < 1 ||
        g->cin % g->groups != 0 || g->cout % g->groups != 0)
        return CONVT3D_ERR_GEOMETRY;
    const int ins[3] = {g->d, g->h, g->w};
    const int64_t lim = (int64_t)INT32_MAX;
    int64_t S = 1, K = 1;
    for (int i = 0; i < 3; ++i) {
        if (g->k[i] < 1 || g->stride[i] < 1 || g->stride[i] > kMaxStride || g->pad[i] < 0 || g->dilation[i] < 1 ||
            g->out_pad[i] < 0 || g->out_pad[i] >= std::max(g->stride[i], g->dilation[i]))
            return CONVT3D_ERR_GEOMETRY;
        if (g->k[i] > 4096 || g->dilation[i] > 4096 || g->pad[i] > lim / 8 || g->out_pad[i] > 4096)
            return CONVT3D_ERR_TOO_LARGE;
        const int64_t o = out_dim(ins[i], g->k[i], g->stride[i], g->pad[i], g->out_pad[i], g->dilation[i]);
        if (o < 1) return CONVT3D_ERR_GEOMETRY;
        if (o > lim / 8) return CONVT3D_ERR_TOO_LARGE;
        S *= o;
        K *= g->k[i];
        if (S > lim || K > lim) return CONVT3D_ERR_TOO_LARGE;
    }
    if ((int64_t)g->n * g->cout * S > lim || (int64_t)g->n * g->cin * g->d * g->h * g->w > lim ||
        (int64_t)g->cin * (g->cout / g->groups) * K > lim / 4)
        return CONVT3D_ERR_TOO_LARGE;
    return CONVT3D_OK;
}

int make_geometry(const convt3d_geom *g, Plan *pl) {
    int st = validate_geom(g);
    if (st) return st;
    pl->g = *g;
    const int ins[3] = {g->d, g->h, g->w};
    int outs[3];
    for (int dim = 0; dim < 3; ++dim) {
        outs[dim] = (int)out_dim(ins[dim], g->k[dim], g->stride[dim], g->pad[dim], g->out_pad[dim], g->dilation[dim]);
        const int s = g->stride[dim], dl = g->dilation[dim], k = g->k[dim], p = g->pad[dim];
        const int gc = gcd_int(dl, s);
        pl->s3[dim] = s;
        pl->ts[dim] = s / gc;
        pl->pe[dim] = dl / gc;
        pl->Q[dim] = (int)ceil_div(outs[dim], s);
        for (int rho = 0; rho < kMaxStride; ++rho) {
            DimPhase &d = pl->ph[dim][rho];
            d = DimPhase{0, 0, 0, 0};
            if (rho >= s) continue;
            d.nq = outs[dim] > rho ? (int)ceil_div(outs[dim] - rho, s) : 0;
            // smallest tap r (< s/g) with dl*r = rho + p (mod s)
            int r = -1;
            for (int t = 0; t < pl->ts[dim] && r < 0; ++t)
                if (((int64_t)dl * t - rho - p) % s == 0) r = t;
            if (r < 0 || r >= k) continue;  // no tap reaches this phase
            d.r = r;
            d.c = (int)floor_div((int64_t)rho + p - (int64_t)dl * r, s);  // exact
            d.J = (int)ceil_div(k - r, pl->ts[dim]);
        }
    }
    pl->Do = outs[0];
    pl->Ho = outs[1];
    pl->Wo = outs[2];
    pl->S = (int64_t)pl->Do * pl->Ho * pl->Wo;
    pl->nph = pl->s3[0] * pl->s3[1] * pl->s3[2];
    pl->G = g->groups;
    pl->cig = g->cin / g->groups;
    pl->cog = g->cout / g->groups;
    pl->cb_total = (int)ceil_div(pl->cog, 32);
    pl->octets = (int)ceil_div(pl->cig, kOctet);
    // Packed weights of one group: for each phase, for each 32-channel output
    // block, the float4 groups ordered (input-channel octet, tap); one group
    // holds, for each of the 64 lanes, the A operands of 4 consecutive MFMA
    // k-steps.  Groups follow one another.
    int64_t off = 0;
    const int sh = pl->s3[1], sw = pl->s3[2];
    for (int ph = 0; ph < pl->nph; ++ph) {
        const int rd = ph / (sh * sw), rh = (ph / sw) % sh, rw = ph % sw;
        const int nt = pl->ph[0][rd].J * pl->ph[1][rh].J * pl->ph[2][rw].J;
        pl->ntaps[ph] = nt;
        pl->steps4[ph] = pl->octets * nt;
        pl->wp_off[ph] = off;
        off += (int64_t)pl->cb_total * pl->steps4[ph] * 64 * 4;
    }
    pl->packed_floats = off;
    if (off * pl->G > (int64_t)INT32_MAX) return CONVT3D_ERR_TOO_LARGE;
    return CONVT3D_OK;
}

static int64_t valid_taps_dim(int out, int in, int k, int s, int p, int dl) {
    int64_t t = 0;
    for (int o = 0; o < out; ++o)
        for (int kk = 0; kk < k; ++kk) {
            const int64_t v = (int64_t)o + p - (int64_t)dl * kk;
            if (v >= 0 && v % s == 0 && v / s < in) ++t;
        }
    return t;
}

static void ws_layout(Plan *pl) {
    const convt3d_geom &g = pl->g;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~size_t(255);
        return o;
    };
    pl->ws_partials = pl->ws_ab = pl->ws_bins = 0;
    const int epi = pl->e.kind;
    if (pl->eval) {
        const EvalGeom &E = pl->eg;
        pl->ws_bins = take((size_t)E.N * E.Cin * E.nchunk * E.nbins * sizeof(float));
    } else if (epi == CONVT3D_EPI_RELU_GROUPNORM || epi == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL) {
        pl->ws_partials = take((size_t)g.n * pl->tiles_per_n * g.cout * 2 * sizeof(float));
        if (epi == CONVT3D_EPI_RELU_GROUPNORM)
            pl->ws_ab = take((size_t)g.n * g.cout * 2 * sizeof(float));
    }
    pl->ws_bytes = off;
}

// Input bins of the evaluation-mode BatchNorm + pool path.  Along one dim,
// tap t reaches output s*i - p + dl*t in [0, out) from inputs i in
// [ceil((p - dl*t)/s), floor((out - 1 + p - dl*t)/s)] clipped to [0, in); the
// cuts are every such range's ends plus 0 and in, so each range is a union of
// consecutive bins.
int make_eval_geom(const convt3d_geom *g, EvalGeom *eg) {
    const int st = validate_geom(g);
    if (st) return st;
    if (g->k[0] > kEvalMaxK || g->k[1] > kEvalMaxK || g->k[2] > kEvalMaxK) return CONVT3D_ERR_UNSUPPORTED;
    std::memset(eg, 0, sizeof(*eg));
    eg->N = g->n; eg->Cin = g->cin; eg->Cout = g->cout;
    eg->cig = g->cin / g->groups; eg->cog = g->cout / g->groups;
    eg->D = g->d; eg->H = g->h; eg->W = g->w;
    const int ins[3] = {g->d, g->h, g->w};
    int64_t S = 1;
    for (int dim = 0; dim < 3; ++dim) {
        const int in = ins[dim], k = g->k[dim], s = g->stride[dim], p = g->pad[dim], dl = g->dilation[dim];
        eg->k3[dim] = k;
        const int out = (int)out_dim(in, k, s, p, g->out_pad[dim], dl);
        S *= out;
        std::vector<int> cuts = {0, in};
        for (int t = 0; t < k; ++t) {
            const int64_t a = (int64_t)p - (int64_t)dl * t, b = (int64_t)out - 1 + p - (int64_t)dl * t;
            const int64_t lo = std::max<int64_t>(ceil_div_any(a, s), 0);
            const int64_t hi = std::min<int64_t>(floor_div(b, s), in - 1);
            if (lo > hi) {
                eg->lo[dim][t] = 1;
                eg->hi1[dim][t] = 0;  // reaches nothing
                continue;
            }
            eg->lo[dim][t] = (int)lo;
            eg->hi1[dim][t] = (int)hi + 1;
            cuts.push_back((int)lo);
            cuts.push_back((int)hi + 1);
        }
        std::sort(cuts.begin(), cuts.end());
        cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
        eg->nb[dim] = (int)cuts.size() - 1;
        for (size_t j = 0; j < cuts.size(); ++j) eg->cut[dim][j] = cuts[j];
    }
    eg->nbins = eg->nb[0] * eg->nb[1] * eg->nb[2];
    eg->inv_S = 1.0 / (double)S;
    if ((int64_t)eg->cig * g->cout * eg->nbins > (int64_t)INT32_MAX / 4) return CONVT3D_ERR_TOO_LARGE;
    // d-chunks: enough workgroups to cover the chip when n * cin is small
    const int64_t planes = std::max<int64_t>((int64_t)g->n * g->cin, 1);
    int64_t nchunk = (kEvalTargetBlocks + planes - 1) / planes;
    nchunk = std::max<int64_t>(1, std::min<int64_t>(nchunk, g->d));
    eg->dchunk = (int)((g->d + nchunk - 1) / nchunk);
    eg->nchunk = (int)((g->d + eg->dchunk - 1) / eg->dchunk);
    if (planes * eg->nchunk > (int64_t)INT32_MAX || planes * eg->nchunk * eg->nbins > (int64_t)INT32_MAX)
        return CONVT3D_ERR_TOO_LARGE;
    return CONVT3D_OK;
}

// Search of the kernel configuration: every (variant, wave grid, border split,
// phase loop, halo buffers) with its best box per region and channel chunk,
// ranked by the cost model.  Returns the best max_k plans, cheapest first.
int plan_candidates(const convt3d_geom *g, const convt3d_epilogue *e, int max_k, std::vector<Plan> *out,
                    const Plan *like) {
    if (!g || !e || !out) return CONVT3D_ERR_NULL;
    out->clear();
    if (max_k < 1) max_k = 1;
    Plan base{};
    Plan *pl = &base;
    int st = make_geometry(g, pl);
    // the conv kernel addresses an output row pair with 32-bit byte offsets
    if (st == CONVT3D_OK && pl->S * 20 >= (int64_t(1) << 32)) st = CONVT3D_ERR_TOO_LARGE;
    if (st) return st;
    pl->e = *e;
    if (e->kind < CONVT3D_EPI_NONE || e->kind > CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL)
        return CONVT3D_ERR_UNSUPPORTED;
    if (e->kind == CONVT3D_EPI_RELU_GROUPNORM && (e->groups < 1 || g->cout % e->groups != 0))
        return CONVT3D_ERR_GROUPS;
    if (e->kind == CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL) {
        // no convolution: one plan, the bin sums of x and their contraction
        st = make_eval_geom(g, &pl->eg);
        if (st) return st;
        pl->eval = 1;
        pl->valid_macs = 0;
        ws_layout(pl);
        out->push_back(*pl);
        return CONVT3D_OK;
    }
    // the conv kernel stages input channel planes through 32-bit buffer offsets
    if ((int64_t)g->d * g->h * g->w > kMaxInputPlane) return CONVT3D_ERR_TOO_LARGE;
    // the in-register softmax needs every channel in one workgroup (<= 4 blocks
    // of 32, one channel group); beyond that the conv stores y and a second
    // pass finishes
    const bool softmax = e->kind == CONVT3D_EPI_SOFTMAX_SIGMOID && pl->cb_total <= 4 && pl->G == 1;
    pl->softmax_pass = e->kind == CONVT3D_EPI_SOFTMAX_SIGMOID && !softmax;
    const bool no_y_store = e->kind == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL;

    const int sd = pl->s3[0], sh = pl->s3[1], sw = pl->s3[2];
    const int ins[3] = {g->d, g->h, g->w};
    // every output channel sums over the cig input channels of its group
    pl->valid_macs = (int64_t)g->n * pl->cig * g->cout *
                     valid_taps_dim(pl->Do, g->d, g->k[0], sd, g->pad[0], g->dilation[0]) *
                     valid_taps_dim(pl->Ho, g->h, g->k[1], sh, g->pad[1], g->dilation[1]) *
                     valid_taps_dim(pl->Wo, g->w, g->k[2], sw, g->pad[2], g->dilation[2]);

    // ---- tiling regions.  Along each dim, positions q whose every phase has all
    // of its taps on the input form the interior [lo, hi); the borders around it
    // have fewer live taps.  Tiling each (border/interior)^3 region with its own
    // box lets border tiles skip the taps that cannot reach the input.
    struct Seg { int a, b; };
    Seg segs_split[3][3], segs_whole[3][1];
    Seg segs_lowonly[3][2], segs_highonly[3][2];  // one border on its own, the other in the interior
    int nseg_split[3];
    for (int dim = 0; dim < 3; ++dim) {
        int lo = 0, hi = pl->Q[dim];
        for (int rho = 0; rho < pl->s3[dim]; ++rho) {
            const DimPhase &d = pl->ph[dim][rho];
            if (d.J == 0) continue;
            lo = std::max(lo, pl->pe[dim] * (d.J - 1) - d.c);
            hi = std::min(hi, ins[dim] - d.c);
        }
        lo = std::min(std::max(lo, 0), pl->Q[dim]);
        hi = std::max(std::min(hi, pl->Q[dim]), lo);
        int &ns = nseg_split[dim];
        ns = 0;
        if (lo > 0) segs_split[dim][ns++] = {0, lo};
        if (hi > lo) segs_split[dim][ns++] = {lo, hi};
        if (pl->Q[dim] > hi) segs_split[dim][ns++] = {hi, pl->Q[dim]};
        segs_whole[dim][0] = {0, pl->Q[dim]};
        segs_lowonly[dim][0] = {0, lo};
        segs_lowonly[dim][1] = {lo, pl->Q[dim]};
        segs_highonly[dim][0] = {0, hi};
        segs_highonly[dim][1] = {hi, pl->Q[dim]};
    }
    // live taps summed over the tiles of a segment for a tile length
    auto seg_live = [&](int dim, int rho, const Seg &sg, int tq) {
        const DimPhase &d = pl->ph[dim][rho];
        if (d.J == 0) return (int64_t)0;
        int64_t t = 0;
        for (int q0 = sg.a; q0 < sg.b; q0 += tq) {
            const int te = std::min(tq, sg.b - q0);
            int lo, hi;
            live_taps(q0, te, d.c, pl->pe[dim], d.J, ins[dim], &lo, &hi);
            if (hi >= lo) t += hi - lo + 1;
        }
        return t;
    };
    // the same along d, each d-tile's live taps weighted by the output columns
    // its workgroup runs MFMAs for: whole waves of wave_cols positions up to
    // the rows the tile has (the kernel skips waves with no tile position)
    auto seg_live_cols = [&](int rho, const Seg &sg, int tq, int plane, int wave_cols, int pt) {
        const DimPhase &d = pl->ph[0][rho];
        if (d.J == 0) return (int64_t)0;
        int64_t t = 0;
        for (int q0 = sg.a; q0 < sg.b; q0 += tq) {
            const int te = std::min(tq, sg.b - q0);
            int lo, hi;
            live_taps(q0, te, d.c, pl->pe[0], d.J, ins[0], &lo, &hi);
            const int64_t cols = std::min<int64_t>(pt, ceil_div((int64_t)te * plane, wave_cols) * wave_cols);
            if (hi >= lo) t += (hi - lo + 1) * cols;
        }
        return t;
    };

    // Optional override for tile sweeps:
    // CONVT3D_PLAN="variant,WCO,TQd,TQh,TQw,CI_T[,split]" restricts the search
    // to that variant / wave grid / chunk, with that box in the largest region
    // and (bit 0 d, 1 h, 2 w) those dims split into border / interior segments,
    // with bit 3 + d (6 + d) set when only the low (high) border of dim d is a
    // segment of its own (ignored if it does not fit).  A negative field leaves that choice free
    // (the box needs all three of TQd, TQh, TQw to be fixed).
    int force[7] = {-1, -1, -1, -1, -1, -1, -1};
    if (const char *env = std::getenv("CONVT3D_PLAN")) {
        const int got = std::sscanf(env, "%d,%d,%d,%d,%d,%d,%d", &force[0], &force[1], &force[2], &force[3],
                                    &force[4], &force[5], &force[6]);
        if (got < 6) force[0] = -1;
    }
    // `like`: only that plan's configuration, every border segmentation
    if (like) {
        force[0] = like->variant; force[1] = like->WCO;
        force[2] = like->TQ[0]; force[3] = like->TQ[1]; force[4] = like->TQ[2];
        force[5] = like->CI_T; force[6] = -1;
    }
    const bool forced = force[0] >= 0;
    int order_env = -1;
    if (const char *env = std::getenv("CONVT3D_ORDER")) order_env = std::atoi(env) ? 1 : 0;
    // CONVT3D_PHASE_LOOP=0|1 restricts the phase-group loop choice (tests, sweeps)
    int ploop_only = -1;
    if (const char *env = std::getenv("CONVT3D_PHASE_LOOP")) ploop_only = std::atoi(env) ? 1 : 0;
    if (like) ploop_only = like->phase_loop;
    // workgroups are planned for every (sample, channel group); an empty batch like n = 1
    const int64_t nn = (int64_t)std::max(g->n, 1) * pl->G;
    const int CI_pad = pl->octets * kOctet;

    std::vector<std::pair<double, Plan>> top;  // cheapest first, at most max_k
    bool found = false, too_large = false;
    for (int vi = 0; vi < kNumVariants; ++vi) {
        const Variant v = kVariants[vi];
        if (sw % v.NPH != 0) continue;
        if (forced && vi != force[0]) continue;
        if (v.softmax != softmax) continue;
        if (softmax && v.CBW < pl->cb_total) continue;
        if (softmax && v.CBW >= 2 * pl->cb_total) continue;  // keep only the tightest fit
        for (int WCO = 1; WCO <= 4; WCO *= 2) {
          const int WPOS = 4 / WCO;
          if (forced && force[1] >= 0 && WCO != force[1]) continue;
          // segments per dim: mode 0 whole, 1 low border / interior / high border,
          // 2 low border / interior + high border, 3 low border + interior / high
          // border (a border's dead taps can cost less than the padding of an
          // interior whose length the box does not divide).  Reported as bit d
          // (dim split), bit 3 + d (mode 2) and bit 6 + d (mode 3).
          for (int modes = 0; modes < 64; ++modes) {
           int split = 0;
           for (int dim = 0; dim < 3; ++dim) {
               const int m = (modes >> (2 * dim)) & 3;
               if (m) split |= 1 << dim;
               if (m == 2) split |= 1 << (3 + dim);
               if (m == 3) split |= 1 << (6 + dim);
           }
           // ploop: one workgroup loops over every (rho_d, rho_h) group on one staged
           // halo (needs the whole channel range in one LDS chunk)
           for (int ploop = 0; ploop < (sd * sh > 1 ? 2 : 1); ++ploop) {
            if (forced && force[6] >= 0 && split != force[6]) continue;
            if (ploop_only >= 0 && ploop != ploop_only) continue;
            if (ploop && !v.phase_loop) continue;
            Seg segs[3][3];
            int nseg[3];
            bool redundant = false;
            for (int dim = 0; dim < 3; ++dim) {
                const int m = (modes >> (2 * dim)) & 3;
                if (m == 1 && nseg_split[dim] == 1) redundant = true;  // same as unsplit
                if (m >= 2 && nseg_split[dim] < 3) redundant = true;   // same as split or unsplit
                const Seg *src = m == 0 ? segs_whole[dim] : m == 1 ? segs_split[dim]
                                 : m == 2 ? segs_lowonly[dim] : segs_highonly[dim];
                nseg[dim] = m == 0 ? 1 : m == 1 ? nseg_split[dim] : 2;
                for (int i = 0; i < nseg[dim]; ++i) segs[dim][i] = src[i];
            }
            if (redundant) continue;
            if (softmax && WCO != 1) continue;
            const int CO_T = WCO * v.CBW;  // co blocks per workgroup
            if (CO_T > pl->cb_total && WCO > 1) continue;  // do not waste whole waves on padding
            const int co_tiles = (int)ceil_div(pl->cb_total, CO_T);
            const int PT = WPOS * v.PBW * 32;
            const int nwg = sw / v.NPH;
            // halo length along a dim of a box for the phases [rho0, rho0 + nr):
            // inputs q + c - e*j of every phase's taps
            auto halo_len = [&](int dim, int TQ, int rho0, int nr) {
                int lo = INT_MAX, hi = INT_MIN;
                for (int rho = rho0; rho < rho0 + nr; ++rho) {
                    const DimPhase &d = pl->ph[dim][rho];
                    if (d.J == 0) continue;
                    lo = std::min(lo, d.c - pl->pe[dim] * (d.J - 1));
                    hi = std::max(hi, TQ - 1 + d.c);
                }
                return lo <= hi ? hi - lo + 1 : 0;
            };
            auto halo_w = [&](int TQw, int wg) { return halo_len(2, TQw, wg * v.NPH, v.NPH); };
            // largest region (the one a forced box applies to)
            int big = 0, big_vol = -1, ri = 0;
            for (int i0 = 0; i0 < nseg[0]; ++i0)
                for (int i1 = 0; i1 < nseg[1]; ++i1)
                    for (int i2 = 0; i2 < nseg[2]; ++i2, ++ri) {
                        const int vol = (segs[0][i0].b - segs[0][i0].a) * (segs[1][i1].b - segs[1][i1].a) *
                                        (segs[2][i2].b - segs[2][i2].a);
                        if (vol > big_vol) { big_vol = vol; big = ri; }
                    }
            // best box per region
            struct RChoice { int box[3], nt[3]; int64_t tiles, issued, staged; int slab; double cost; };
            RChoice rc[kMaxRegions];
            int nreg = 0;
            bool ok_all = true;
            for (int i0 = 0; i0 < nseg[0] && ok_all; ++i0)
                for (int i1 = 0; i1 < nseg[1] && ok_all; ++i1)
                    for (int i2 = 0; i2 < nseg[2] && ok_all; ++i2) {
                        const Seg sgd = segs[0][i0], sgh = segs[1][i1], sgw = segs[2][i2];
                        const int ext[3] = {sgd.b - sgd.a, sgh.b - sgh.a, sgw.b - sgw.a};
                        RChoice bestr{};
                        bestr.cost = 1e300;
                        // rows of at least 16 positions keep LDS reads and stores contiguous;
                        // the BatchNorm-pool epilogue stores no y, so its boxes may be narrower
                        // (a 1-wide box gives a w border its exact taps)
                        const int TQw_min = no_y_store ? 1 : std::min(ext[2], 16);
                        for (int TQw = TQw_min; TQw <= std::min(ext[2], PT); ++TQw) {
                            for (int TQh = 1; TQh <= std::min(ext[1], PT / TQw); ++TQh) {
                                // boxes that leave a whole position block empty are skipped
                                // unless the box cannot grow any more along d
                                const int maxd = std::min(ext[0], PT / (TQw * TQh));
                                int mind = std::max(1, (PT - 32) / (TQw * TQh));
                                if (mind > maxd) mind = maxd;
                                for (int TQd = mind; TQd <= maxd; ++TQd) {
                                    if (forced && nreg == big && force[2] >= 0 && force[3] >= 0 && force[4] >= 0 &&
                                        (TQd != force[2] || TQh != force[3] || TQw != force[4]))
                                        continue;
                                    int HD = 1, HH = 1, HW = TQw;
                                    if (ploop) {  // union of the groups' footprints
                                        HD = halo_len(0, TQd, 0, sd);
                                        HH = halo_len(1, TQh, 0, sh);
                                        if (HD == 0) HD = TQd;
                                        if (HH == 0) HH = TQh;
                                    } else {
                                        for (int rho = 0; rho < sd; ++rho) HD = std::max(HD, halo_len(0, TQd, rho, 1));
                                        for (int rho = 0; rho < sh; ++rho) HH = std::max(HH, halo_len(1, TQh, rho, 1));
                                        HD = std::max(HD, TQd);
                                        HH = std::max(HH, TQh);
                                    }
                                    for (int wg = 0; wg < nwg; ++wg) HW = std::max(HW, halo_w(TQw, wg));
                                    const int slab = HD * HH * HW;
                                    if ((int64_t)(ploop ? CI_pad : kOctet) * slab * 4 > kMaxLdsBytes) continue;
                                    const int nt[3] = {(int)ceil_div(ext[0], TQd), (int)ceil_div(ext[1], TQh),
                                                       (int)ceil_div(ext[2], TQw)};
                                    const int64_t tiles = (int64_t)nt[0] * nt[1] * nt[2];
                                    int64_t taps = 0, halo = 0;
                                    for (int rd = 0; rd < sd; ++rd) {
                                        const int64_t ld = seg_live_cols(rd, sgd, TQd, TQh * TQw, v.PBW * 32, PT);
                                        for (int rh = 0; rh < sh; ++rh) {
                                            const int64_t lh = seg_live(1, rh, sgh, TQh);
                                            int64_t lw = 0;
                                            for (int rw = 0; rw < sw; ++rw) lw += seg_live(2, rw, sgw, TQw);
                                            taps += ld * lh * lw;
                                            if (ploop || pl->ph[0][rd].J == 0 || pl->ph[1][rh].J == 0) continue;
                                            for (int wg = 0; wg < nwg; ++wg)
                                                halo += (int64_t)halo_len(0, TQd, rd, 1) * halo_len(1, TQh, rh, 1) *
                                                        halo_w(TQw, wg);
                                        }
                                    }
                                    // taps already carries the live output columns of each tile
                                    const int64_t issued = nn * co_tiles * CO_T * 32 * CI_pad * taps;
                                    const int64_t staged = nn * co_tiles * tiles * CI_pad * halo;
                                    if (ploop)
                                        for (int wg = 0; wg < nwg; ++wg) halo += (int64_t)HD * HH * halo_w(TQw, wg);
                                    const int64_t wgs = nn * co_tiles * sd * sh * nwg * tiles;
                                    // MAC-equivalents: issued MFMA work, ~24 per staged element
                                    // (address arithmetic, load, LDS store), ~64 per output of
                                    // the epilogue
                                    double cost = (double)issued + 24.0 * (double)staged +
                                                  (double)wgs * CO_T * 32 * PT * v.NPH * 64.0;
                                    // rows that break inside a 32-position block split its
                                    // stores into more memory segments
                                    if (32 % TQw != 0 && TQw % 32 != 0) cost *= 1.05;
                                    if (cost < bestr.cost) {
                                        bestr.cost = cost;
                                        bestr.box[0] = TQd; bestr.box[1] = TQh; bestr.box[2] = TQw;
                                        for (int i = 0; i < 3; ++i) bestr.nt[i] = nt[i];
                                        bestr.tiles = tiles;
                                        bestr.issued = issued;
                                        bestr.staged = staged;
                                        bestr.slab = slab;
                                    }
                                }
                            }
                        }
                        if (bestr.cost >= 1e300) { ok_all = false; break; }
                        rc[nreg++] = bestr;
                    }
            if (!ok_all) continue;
            int max_slab = 0;
            int64_t tiles_total = 0, issued = 0;
            double cost_regions = 0.0;
            for (int r = 0; r < nreg; ++r) {
                max_slab = std::max(max_slab, rc[r].slab);
                tiles_total += rc[r].tiles;
                issued += rc[r].issued;
                cost_regions += rc[r].cost;
            }
            // LDS of a workgroup for a channel chunk: the halo (rounded to 256
            // floats), then the reduction scratch
            const int red_floats = WPOS * CO_T * 32 * 2;
            auto halo_floats = [&](int ci_t) { return (int)ceil_div((int64_t)ci_t * max_slab, 256) * 256; };
            auto lds_of = [&](int ci_t) { return (int64_t)(halo_floats(ci_t) + red_floats) * 4; };
            // largest channel chunk whose LDS still lets the register-limited number
            // of workgroups share a CU (measured: occupancy beats fewer barriers)
            int CI_T = 0;
            for (int m = 4; m >= 1; m /= 2) {
                if (pl->octets % m != 0) continue;  // chunks never pass the packed octets
                const int64_t bytes = lds_of(m * kOctet);
                if (bytes > kMaxLdsBytes) continue;
                if (m > 1 && bytes * v.waves_per_simd > 160 * 1024) continue;
                CI_T = m * kOctet;
                break;
            }
            if (ploop) CI_T = lds_of(CI_pad) <= kMaxLdsBytes ? CI_pad : 0;
            if (forced && force[5] > 0) {
                if (force[5] % kOctet || pl->octets % (force[5] / kOctet) || lds_of(force[5]) > kMaxLdsBytes)
                    continue;
                CI_T = force[5];
            }
            if (v.prefetch) {
                // one octet per chunk whose halo fits kRpPositions per thread, 32-bit
                // plane offsets, and a further chunk to prefetch
                if (pl->octets < 2 || max_slab > kRpPositions * kBlockThreads ||
                    (int64_t)kOctet * g->d * g->h * g->w > kMaxChunkPlanes ||
                    (forced && force[5] > 0 && force[5] != kOctet))
                    continue;
                CI_T = lds_of(kOctet) <= kMaxLdsBytes ? kOctet : 0;
            }
            if (CI_T == 0) continue;
            const int nchunks = (int)ceil_div(CI_pad, CI_T);
            const int64_t grid = nn * co_tiles * (ploop ? 1 : sd * sh) * nwg * tiles_total;
            // whole rounds of workgroups over the CUs; workgroups per CU from the
            // variant's register occupancy and the LDS size
            const int lds_wg = (int)lds_of(CI_T);
            const int per_cu = std::max(1, std::min(v.waves_per_simd, 160 * 1024 / lds_wg));
            const double slots = 256.0 * per_cu;
            const double rounds = std::ceil((double)grid / slots);
            // exposed staging waits: co-resident workgroups advance in lockstep on
            // the shared MFMA pipe, so a stage idles the CU (measured about 2000 CU
            // cycles = 250k MAC-equivalents per chunk and workgroup)
            // (a prefetching kernel waits in full only for its first chunk)
            const double waits = v.prefetch ? 1.0 + 0.25 * (nchunks - 1) : (double)nchunks;
            double cost = cost_regions + (double)grid * kStageWaitMacs * waits;
            cost *= rounds * slots / (double)grid;
            // few waves per SIMD hide less latency; fewer MFMA tiles per wave mean
            // more operand traffic per MFMA
            // (measured on MI355X: 3 workgroups per CU reach ~67% MFMA busy, 2 ~60%)
            cost *= per_cu == 1 ? 1.35 : per_cu == 2 ? 1.15 : per_cu == 3 ? 1.04 : 1.0;
            cost *= 1.0 + 0.15 / (v.CBW * v.PBW * v.NPH);
            // measured: splitting the output channels over fewer waves (WCO < 4)
            // costs MFMA issue rate when the channels could fill four waves
            if (!softmax && WCO < 4 && pl->cb_total >= 4) cost *= WCO == 2 ? 1.1 : 1.2;
            if ((int)top.size() < max_k || cost < top.back().first) {
                found = true;
                Plan c = *pl;
                c.variant = vi;
                c.CBW = v.CBW; c.NPH = v.NPH; c.PBW = v.PBW;
                c.WCO = WCO; c.WPOS = WPOS;
                c.nreg = nreg;
                int64_t off = 0;
                int r = 0;
                for (int i0 = 0; i0 < nseg[0]; ++i0)
                    for (int i1 = 0; i1 < nseg[1]; ++i1)
                        for (int i2 = 0; i2 < nseg[2]; ++i2, ++r) {
                            const Seg sg[3] = {segs[0][i0], segs[1][i1], segs[2][i2]};
                            for (int dim = 0; dim < 3; ++dim) {
                                c.rg[r][dim] = sg[dim].a;
                                c.rg[r][3 + dim] = sg[dim].b;
                                c.rg[r][6 + dim] = rc[r].box[dim];
                                c.rg[r][9 + dim] = rc[r].nt[dim];
                            }
                            c.rg_off[r] = (int)off;
                            off += rc[r].tiles;
                        }
                c.rg_off[nreg] = (int)off;
                c.tiles_total = (int)tiles_total;
                for (int dim = 0; dim < 3; ++dim) c.TQ[dim] = rc[big].box[dim];
                c.CI_T = CI_T; c.nchunks = nchunks;
                c.phase_loop = ploop;
                c.split = split;
                c.red_off = halo_floats(CI_T);
                c.lds_bytes = lds_wg;
                c.co_tiles = co_tiles; c.nwgroups = nwg;
                c.tiles_per_n = (int64_t)sd * sh * nwg * tiles_total;
                c.grid_x = tiles_total;
                c.grid_y = (int64_t)co_tiles * (ploop ? 1 : sd * sh) * nwg;
                // one launch for every (sample, group) unless that passes the
                // grid's z limit: then one launch per group
                c.group_launch = (int64_t)g->n * pl->G <= 65535 ? 1 : 0;
                c.grid_z = c.group_launch ? (int64_t)g->n * pl->G : g->n;
                c.issued_macs = issued / nn * g->n * pl->G;  // every channel group
                // packed weights that do not fit in half an L2: keep each XCD on
                // one (co tile, phase) group at a time (CONVT3D_ORDER overrides)
                c.order = (c.grid_y > 1 && pl->packed_floats * 4 > kL2Bytes / 2) ? 1 : 0;
                if (order_env >= 0) c.order = order_env;
                // the kernel forms a linear workgroup index in 32-bit arithmetic
                if (c.grid_x > INT32_MAX || c.grid_y > 65535 || c.grid_z > 65535 ||
                    c.grid_x * c.grid_y * c.grid_z > INT32_MAX) {
                    too_large = true;
                    continue;
                }
                ws_layout(&c);
                // one entry per kernel configuration (variant, wave grid, box,
                // chunk, phase loop): plans that differ only in how the borders
                // are segmented run within noise of each other, so the timed
                // candidates should spread over configurations instead
                bool dominated = false;
                for (auto it = top.begin(); it != top.end() && !like; ++it) {
                    const Plan &o = it->second;
                    if (o.variant != c.variant || o.WCO != c.WCO || o.CI_T != c.CI_T ||
                        o.phase_loop != c.phase_loop || o.TQ[0] != c.TQ[0] || o.TQ[1] != c.TQ[1] ||
                        o.TQ[2] != c.TQ[2])
                        continue;
                    if (it->first <= cost) dominated = true;
                    else top.erase(it);
                    break;
                }
                if (dominated) continue;
                auto at = top.begin();
                while (at != top.end() && at->first <= cost) ++at;
                top.insert(at, std::make_pair(cost, c));
                if ((int)top.size() > max_k) top.pop_back();
            }
           }
          }
        }
    }
    if (!found) return CONVT3D_ERR_UNSUPPORTED;
    if (top.empty()) return too_large ? CONVT3D_ERR_TOO_LARGE : CONVT3D_ERR_UNSUPPORTED;
    for (auto &t : top) out->push_back(t.second);
    return CONVT3D_OK;
}

// Chunks per row of the statistics pass over a conv output in memory (each
// workgroup sums kRowStatChunk vectors of a row: float4 when the row length
// is a multiple of 4, else float).
int row_stat_chunks(int64_t S) {
    const int64_t len = S % 4 == 0 ? S / 4 : S;
    const int64_t c = (len + kRowStatChunk - 1) / kRowStatChunk;
    return (int)(c < 1 ? 1 : c);
}

int make_plan(const convt3d_geom *g, const convt3d_epilogue *e, Plan *pl) {
    std::vector<Plan> c;
    const int st = plan_candidates(g, e, 1, &c);
    if (st) return st;
    *pl = c[0];
    return CONVT3D_OK;
}

void fill_conv_params(const Plan &pl, ConvParams *cp) {
    std::memset(cp, 0, sizeof(*cp));
    const convt3d_geom &g = pl.g;
    cp->N = g.n; cp->Cin = pl.cig; cp->Cout = pl.cog;
    cp->Cout_total = g.cout;
    cp->x_nstride = g.cin * g.d * g.h * g.w;
    cp->G = pl.group_launch ? pl.G : 1;
    cp->xg = pl.cig * g.d * g.h * g.w;
    cp->wpg = (int)pl.packed_floats;
    cp->D = g.d; cp->H = g.h; cp->W = g.w;
    cp->Do = pl.Do; cp->Ho = pl.Ho; cp->Wo = pl.Wo;
    for (int dim = 0; dim < 3; ++dim) {
        cp->s3[dim] = pl.s3[dim];
        cp->pe[dim] = pl.pe[dim];
    }
    cp->Qd = pl.Q[0]; cp->Qh = pl.Q[1]; cp->Qw = pl.Q[2];
    cp->nreg = pl.nreg;
    for (int r = 0; r < kMaxRegions; ++r)
        for (int i = 0; i < 12; ++i) cp->rg[r][i] = pl.rg[r][i];
    for (int r = 0; r <= kMaxRegions; ++r) cp->rg_off[r] = pl.rg_off[r];
    cp->tiles_total = pl.tiles_total;
    cp->CI_T = pl.CI_T; cp->octets = pl.octets; cp->nchunks = pl.nchunks;
    cp->plane_desc = (int64_t)pl.CI_T * pl.g.d * pl.g.h * pl.g.w > kMaxChunkPlanes;
    cp->cb_total = pl.cb_total;
    cp->WCO = pl.WCO; cp->WPOS = pl.WPOS;
    cp->co_tiles = pl.co_tiles; cp->nwgroups = pl.nwgroups;

    cp->order = pl.order;
    cp->phase_loop = pl.phase_loop; cp->red_off = pl.red_off;
    cp->epi = pl.softmax_pass ? CONVT3D_EPI_NONE : pl.e.kind;
    // GroupNorm needs only per-group sums: when every group is a run of whole
    // 8-channel blocks (and no block straddles a channel-group boundary), the
    // conv epilogue sums each block before the cross-lane reduction
    cp->gn_block8 = pl.e.kind == CONVT3D_EPI_RELU_GROUPNORM && pl.e.groups > 0 &&
                    (pl.g.cout / pl.e.groups) % 8 == 0 && pl.cog % 8 == 0;
    cp->scale = pl.e.kind == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL ? pl.e.scale : 1.0f;
    cp->tiles_per_n = (int)pl.tiles_per_n;
    for (int dim = 0; dim < 3; ++dim)
        for (int r = 0; r < kMaxStride; ++r) {
            cp->pr[dim][r] = pl.ph[dim][r].r;
            cp->pc[dim][r] = pl.ph[dim][r].c;
            cp->pJ[dim][r] = pl.ph[dim][r].J;
        }
    for (int ph = 0; ph < kMaxPhases; ++ph) {
        cp->ntaps[ph] = pl.ntaps[ph];
        cp->wp_off[ph] = (int)pl.wp_off[ph];
        cp->steps4[ph] = pl.steps4[ph];
    }
}

}  // namespace convt3d
