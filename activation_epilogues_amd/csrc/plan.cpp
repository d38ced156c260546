// Host-side planner of libconvt3d: geometry checks, stride-phase tables,
// packed-weight layout, tile choice and workspace layout.
//
// Stride-phase split (p49 page, its gather relation: output o receives tap k
// iff (o + pad - k) is a multiple of the stride, from input (o + pad - k)/s).
// Writing o = s*q + rho, the taps that reach o are k = r + s*j with
// r = (rho + pad) mod s, from input i = q + c - j with c = (rho + pad) div s,
// j = 0 .. J-1, J = ceil((k - r)/s).  Each phase (rho_d, rho_h, rho_w) is a
// dense correlation over q with a J_d x J_h x J_w sub-kernel, so no tap that
// can never be valid is ever multiplied.
#include <algorithm>
#include <climits>
#include <cstring>
#include <vector>

#include "convt3d_internal.hpp"

namespace convt3d {

// Kernel variants compiled into the library (co-blocks per wave, w-phases per
// wave, position blocks per wave).  Keep in sync with the instantiations in
// kernels.hip.
const Variant kVariants[] = {
    {1, 1, 8}, {1, 1, 4}, {1, 1, 2},
    {1, 2, 4}, {1, 2, 2},
    {2, 1, 4}, {2, 2, 2},
    {4, 1, 2}, {4, 2, 1},
};
const int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int64_t out_dim(int64_t in, int64_t k, int64_t s, int64_t p, int64_t op) {
    return (in - 1) * s - 2 * p + k + op;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate_geom(const convt3d_geom *g) {
    if (!g) return CONVT3D_ERR_NULL;
    if (g->n < 0 || g->cin < 1 || g->cout < 1 || g->d < 1 || g->h < 1 || g->w < 1 || g->k < 1 ||
        g->stride < 1 || g->stride > kMaxStride || g->pad < 0 || g->out_pad < 0 ||
        g->out_pad >= g->stride)
        return CONVT3D_ERR_GEOMETRY;
    const int64_t Do = out_dim(g->d, g->k, g->stride, g->pad, g->out_pad);
    const int64_t Ho = out_dim(g->h, g->k, g->stride, g->pad, g->out_pad);
    const int64_t Wo = out_dim(g->w, g->k, g->stride, g->pad, g->out_pad);
    if (Do < 1 || Ho < 1 || Wo < 1) return CONVT3D_ERR_GEOMETRY;
    const int64_t lim = (int64_t)INT32_MAX;
    const int64_t S = Do * Ho * Wo;
    if ((int64_t)g->n * g->cout * S > lim || (int64_t)g->n * g->cin * g->d * g->h * g->w > lim ||
        (int64_t)g->cin * g->cout * g->k * g->k * g->k > lim / 4 || Do > lim / 8 || Ho > lim / 8 ||
        Wo > lim / 8)
        return CONVT3D_ERR_TOO_LARGE;
    return CONVT3D_OK;
}

int make_geometry(const convt3d_geom *g, Plan *pl) {
    int st = validate_geom(g);
    if (st) return st;
    pl->g = *g;
    pl->s = g->stride;
    pl->Do = (int)out_dim(g->d, g->k, g->stride, g->pad, g->out_pad);
    pl->Ho = (int)out_dim(g->h, g->k, g->stride, g->pad, g->out_pad);
    pl->Wo = (int)out_dim(g->w, g->k, g->stride, g->pad, g->out_pad);
    pl->S = (int64_t)pl->Do * pl->Ho * pl->Wo;
    const int s = pl->s;
    const int outs[3] = {pl->Do, pl->Ho, pl->Wo};
    for (int dim = 0; dim < 3; ++dim) {
        pl->Q[dim] = (int)ceil_div(outs[dim], s);
        for (int rho = 0; rho < kMaxStride; ++rho) {
            DimPhase &d = pl->ph[dim][rho];
            if (rho >= s) { d = DimPhase{0, 0, 0, 0}; continue; }
            d.r = (rho + g->pad) % s;
            d.c = (rho + g->pad) / s;
            d.J = d.r < g->k ? (int)ceil_div(g->k - d.r, s) : 0;
            d.nq = outs[dim] > rho ? (int)ceil_div(outs[dim] - rho, s) : 0;
        }
    }
    pl->cb_total = (int)ceil_div(g->cout, 32);
    pl->octets = (int)ceil_div(g->cin, kOctet);
    // Packed weights: for each phase, for each 32-channel output block, the
    // float4 groups ordered (input-channel octet, tap); one group holds, for
    // each of the 64 lanes, the A operands of 4 consecutive MFMA k-steps.
    int64_t off = 0;
    for (int ph = 0; ph < s * s * s; ++ph) {
        const int rd = ph / (s * s), rh = (ph / s) % s, rw = ph % s;
        const int nt = pl->ph[0][rd].J * pl->ph[1][rh].J * pl->ph[2][rw].J;
        pl->ntaps[ph] = nt;
        pl->steps4[ph] = pl->octets * nt;
        pl->wp_off[ph] = off;
        off += (int64_t)pl->cb_total * pl->steps4[ph] * 64 * 4;
    }
    pl->packed_floats = off;
    if (off > (int64_t)INT32_MAX) return CONVT3D_ERR_TOO_LARGE;
    return CONVT3D_OK;
}

// Taps of a phase that touch the input for a tile starting at q0 (tile length
// tq, q extent Q), along one dim: count of j in [max(0, q0+c-(in-1)),
// min(J-1, q0+tq_eff-1+c)].
static int live_taps(const DimPhase &d, int q0, int tq, int Q, int in) {
    if (d.J == 0) return 0;
    const int te = std::min(tq, Q - q0);
    const int lo = std::max(0, q0 + d.c - (in - 1));
    const int hi = std::min(d.J - 1, q0 + te - 1 + d.c);
    return hi >= lo ? hi - lo + 1 : 0;
}

static int64_t sum_live(const DimPhase &d, int tq, int Q, int in) {
    int64_t t = 0;
    for (int q0 = 0; q0 < Q; q0 += tq) t += live_taps(d, q0, tq, Q, in);
    return t;
}

static int64_t valid_taps_dim(int out, int in, int k, int s, int p) {
    int64_t t = 0;
    for (int o = 0; o < out; ++o)
        for (int kk = 0; kk < k; ++kk) {
            const int v = o + p - kk;
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
    pl->ws_partials = pl->ws_ab = 0;
    const int epi = pl->e.kind;
    if (epi == CONVT3D_EPI_RELU_GROUPNORM || epi == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL) {
        pl->ws_partials = take((size_t)g.n * pl->tiles_per_n * g.cout * 2 * sizeof(float));
        if (epi == CONVT3D_EPI_RELU_GROUPNORM)
            pl->ws_ab = take((size_t)g.n * g.cout * 2 * sizeof(float));
    }
    pl->ws_bytes = off;
}

int make_plan(const convt3d_geom *g, const convt3d_epilogue *e, Plan *pl) {
    if (!g || !e) return CONVT3D_ERR_NULL;
    *pl = Plan{};
    int st = make_geometry(g, pl);
    if (st) return st;
    pl->e = *e;
    if (e->kind < CONVT3D_EPI_NONE || e->kind > CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL)
        return CONVT3D_ERR_UNSUPPORTED;
    if (e->kind == CONVT3D_EPI_RELU_GROUPNORM && (e->groups < 1 || g->cout % e->groups != 0))
        return CONVT3D_ERR_GROUPS;
    const bool softmax = e->kind == CONVT3D_EPI_SOFTMAX_SIGMOID;
    if (softmax && pl->cb_total > 4) return CONVT3D_ERR_UNSUPPORTED;

    const int s = pl->s;
    const int ins[3] = {g->d, g->h, g->w};
    pl->valid_macs = (int64_t)g->n * g->cin * g->cout *
                     valid_taps_dim(pl->Do, g->d, g->k, s, g->pad) *
                     valid_taps_dim(pl->Ho, g->h, g->k, s, g->pad) *
                     valid_taps_dim(pl->Wo, g->w, g->k, s, g->pad);

    // sum over tiles of live taps, per (dim, phase, tile length)
    const int tqmax = 4 * 8 * 32;
    std::vector<int64_t> live[3][kMaxStride];
    for (int dim = 0; dim < 3; ++dim)
        for (int rho = 0; rho < s; ++rho) {
            live[dim][rho].assign(std::min(pl->Q[dim], tqmax) + 1, 0);
            for (int tq = 1; tq < (int)live[dim][rho].size(); ++tq)
                live[dim][rho][tq] = sum_live(pl->ph[dim][rho], tq, pl->Q[dim], ins[dim]);
        }

    double best = 1e300;
    Plan bestp = *pl;
    bool found = false;
    for (int vi = 0; vi < kNumVariants; ++vi) {
        const Variant v = kVariants[vi];
        if (s % v.NPH != 0) continue;
        if (softmax && v.CBW < pl->cb_total) continue;
        if (softmax && v.CBW >= 2 * pl->cb_total) continue;  // keep only the tightest fit
        for (int WCO = 1; WCO <= 4; WCO *= 2) {
            const int WPOS = 4 / WCO;
            if (softmax && WCO != 1) continue;
            const int CO_T = WCO * v.CBW;  // co blocks per workgroup
            if (CO_T > pl->cb_total && WCO > 1) continue;  // do not waste whole waves on padding
            const int co_tiles = (int)ceil_div(pl->cb_total, CO_T);
            const int PT = WPOS * v.PBW * 32;
            const int nwg = s / v.NPH;
            // halo extents along w over each group of NPH w-phases
            // rows of at least 16 positions keep LDS reads and output stores contiguous
            const int TQw_min = std::min(pl->Q[2], 16);
            for (int TQw = TQw_min; TQw <= std::min(pl->Q[2], PT); ++TQw) {
                for (int TQh = 1; TQh <= std::min(pl->Q[1], PT / TQw); ++TQh) {
                    // boxes that leave a whole position block empty are skipped unless
                    // the box cannot grow any more along d
                    const int maxd = std::min(pl->Q[0], PT / (TQw * TQh));
                    int mind = std::max(1, (PT - 32) / (TQw * TQh));
                    if (mind > maxd) mind = maxd;
                    for (int TQd = mind; TQd <= maxd; ++TQd) {
                        // LDS halo size (max over phases)
                        int HD = 1, HH = 1, HW = TQw;
                        for (int rho = 0; rho < s; ++rho) {
                            HD = std::max(HD, TQd + std::max(pl->ph[0][rho].J, 1) - 1);
                            HH = std::max(HH, TQh + std::max(pl->ph[1][rho].J, 1) - 1);
                        }
                        for (int wg = 0; wg < nwg; ++wg) {
                            int lo = INT_MAX, hi = INT_MIN;
                            for (int p = 0; p < v.NPH; ++p) {
                                const DimPhase &d = pl->ph[2][wg * v.NPH + p];
                                if (d.J == 0) continue;
                                lo = std::min(lo, d.c - d.J + 1);
                                hi = std::max(hi, TQw - 1 + d.c);
                            }
                            if (lo <= hi) HW = std::max(HW, hi - lo + 1);
                        }
                        const int HWp = HW;
                        const int slab = HD * HH * HWp;
                        int CI_T = 0;
                        for (int m = 4; m >= 1; m /= 2) {
                            if (pl->octets % m != 0) continue;  // chunks never pass the packed octets
                            if ((int64_t)m * kOctet * slab * 4 <= kMaxLdsBytes) { CI_T = m * kOctet; break; }
                        }
                        if (CI_T == 0) continue;
                        const int nchunks = (int)ceil_div(pl->octets * kOctet, CI_T);
                        const int ntile[3] = {(int)ceil_div(pl->Q[0], TQd), (int)ceil_div(pl->Q[1], TQh),
                                              (int)ceil_div(pl->Q[2], TQw)};
                        // issued MACs: per workgroup CO_T*32 x PT x CI_pad x sum_p live taps
                        int64_t taps = 0;
                        for (int rd = 0; rd < s; ++rd) {
                            const int64_t ld = live[0][rd][TQd];
                            for (int rh = 0; rh < s; ++rh) {
                                const int64_t lh = live[1][rh][TQh];
                                int64_t lw = 0;
                                for (int rw = 0; rw < s; ++rw)
                                    lw += live[2][rw][TQw];
                                taps += ld * lh * lw;
                            }
                        }
                        const int64_t nn = std::max(g->n, 1);  // plan an empty batch like n = 1
                        const int64_t issued = nn * co_tiles * CO_T * 32 * PT *
                                               (int64_t)nchunks * CI_T * taps;
                        const int64_t grid = nn * co_tiles * s * s * nwg *
                                             ntile[0] * ntile[1] * ntile[2];
                        // input elements staged into LDS by all workgroups (halo per phase group)
                        int64_t staged = 0;
                        for (int rd = 0; rd < s; ++rd)
                            for (int rh = 0; rh < s; ++rh)
                                for (int wg = 0; wg < nwg; ++wg) {
                                    int lo = INT_MAX, hi = INT_MIN;
                                    for (int p = 0; p < v.NPH; ++p) {
                                        const DimPhase &d = pl->ph[2][wg * v.NPH + p];
                                        if (d.J == 0) continue;
                                        lo = std::min(lo, d.c - d.J + 1);
                                        hi = std::max(hi, TQw - 1 + d.c);
                                    }
                                    if (lo > hi || pl->ph[0][rd].J == 0 || pl->ph[1][rh].J == 0) continue;
                                    staged += (int64_t)(TQd + pl->ph[0][rd].J - 1) * (TQh + pl->ph[1][rh].J - 1) *
                                              (hi - lo + 1);
                                }
                        staged *= nn * co_tiles * (int64_t)ntile[0] * ntile[1] * ntile[2] * nchunks * CI_T;
                        // cost in MAC-equivalents: issued MFMA work, ~24 per staged element
                        // (address arithmetic, load, LDS store), ~64 per output of the epilogue
                        double cost = (double)issued + 24.0 * (double)staged +
                                      (double)grid * CO_T * 32 * PT * v.NPH * 64.0;
                        const double fill = std::min(1.0, (double)grid / 512.0);
                        cost /= fill;
                        if (cost < best) {
                            best = cost;
                            found = true;
                            Plan c = *pl;
                            c.variant = vi;
                            c.CBW = v.CBW; c.NPH = v.NPH; c.PBW = v.PBW;
                            c.WCO = WCO; c.WPOS = WPOS;
                            c.TQ[0] = TQd; c.TQ[1] = TQh; c.TQ[2] = TQw;
                            for (int i = 0; i < 3; ++i) c.ntile[i] = ntile[i];
                            c.CI_T = CI_T; c.nchunks = nchunks;
                            c.HWp = HWp; c.CISTR = slab;
                            c.lds_bytes = CI_T * slab * 4;
                            c.co_tiles = co_tiles; c.nwgroups = nwg;
                            c.tiles_per_n = (int64_t)s * s * nwg * ntile[0] * ntile[1] * ntile[2];
                            c.grid_x = (int64_t)ntile[0] * ntile[1] * ntile[2];
                            c.grid_y = (int64_t)co_tiles * s * s * nwg;
                            c.grid_z = g->n;
                            c.issued_macs = issued / nn * g->n;
                            bestp = c;
                        }
                    }
                }
            }
        }
    }
    if (!found) return CONVT3D_ERR_UNSUPPORTED;
    // the reduction scratch of the epilogue reuses the halo LDS
    const int red = bestp.WPOS * bestp.WCO * bestp.CBW * 32 * 2 * 4;
    bestp.lds_bytes = std::max(bestp.lds_bytes, red);
    if (bestp.grid_x > INT32_MAX || bestp.grid_y > 65535 || bestp.grid_z > 65535)
        return CONVT3D_ERR_TOO_LARGE;
    *pl = bestp;
    ws_layout(pl);
    return CONVT3D_OK;
}

void fill_conv_params(const Plan &pl, ConvParams *cp) {
    std::memset(cp, 0, sizeof(*cp));
    const convt3d_geom &g = pl.g;
    cp->N = g.n; cp->Cin = g.cin; cp->Cout = g.cout;
    cp->D = g.d; cp->H = g.h; cp->W = g.w;
    cp->Do = pl.Do; cp->Ho = pl.Ho; cp->Wo = pl.Wo;
    cp->s = pl.s;
    cp->Qd = pl.Q[0]; cp->Qh = pl.Q[1]; cp->Qw = pl.Q[2];
    cp->TQd = pl.TQ[0]; cp->TQh = pl.TQ[1]; cp->TQw = pl.TQ[2];
    cp->ntd = pl.ntile[0]; cp->nth = pl.ntile[1]; cp->ntw = pl.ntile[2];
    cp->CI_T = pl.CI_T; cp->octets = pl.octets; cp->nchunks = pl.nchunks;
    cp->cb_total = pl.cb_total;
    cp->WCO = pl.WCO; cp->WPOS = pl.WPOS;
    cp->co_tiles = pl.co_tiles; cp->nwgroups = pl.nwgroups;
    cp->HWp = pl.HWp; cp->CISTR = pl.CISTR;
    cp->epi = pl.e.kind;
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
