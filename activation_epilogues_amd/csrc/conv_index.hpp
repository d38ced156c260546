// Index arithmetic of convt3d_mfma_kernel (kernels.hip): which work item a
// workgroup runs, the tile box and its input halo, the live tap ranges, and
// the LDS, packed-weight, output and partial-sum offsets.  The kernel calls
// these functions; a host build of the same header replays every workgroup's
// and lane's addresses on the CPU against the buffer sizes (tests), so the
// bounds that test checks are those of the kernel's own arithmetic.
#pragma once

#include <climits>

#include "convt3d_internal.hpp"

#if defined(__HIP__)
#define CONVT3D_IX __host__ __device__ __forceinline__
#else
#define CONVT3D_IX inline
#endif

namespace convt3d {
namespace ix {

CONVT3D_IX int imin(int a, int b) { return a < b ? a : b; }
CONVT3D_IX int imax(int a, int b) { return a > b ? a : b; }

// floor / ceil of a / b for b > 0 and any sign of a (tap ranges with
// dilation; b is wave-uniform: 1 without dilation, a power of two for the
// usual dilations, where an arithmetic shift is the floor)
CONVT3D_IX int floor_div_any(int a, int b) {
    if (b == 1) return a;
    if ((b & (b - 1)) == 0) return a >> __builtin_ctz((unsigned)b);
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}
CONVT3D_IX int ceil_div_any(int a, int b) { return -floor_div_any(-a, b); }

// ---- workgroup -> work item.  Workgroups are handed to the XCDs round-robin
// (dispatch index i runs on XCD i % kNumXcd), each XCD with its own L2.  The
// dispatch index bid is mapped to a linear work index so that every XCD gets
// one contiguous range; the halo overlap of neighbouring tiles then hits in
// one L2.  Within it either the (co tile, phase) index varies fastest (those
// workgroups read the same input box; order 0) or the tile does (an XCD keeps
// to one phase's weights when all of them do not fit in its L2; order 1); the
// (sample, channel group) index varies slowest.
struct WorkItem {
    int bx;       // tile index over all regions, [0, tiles_total)
    int co_tile;  // output-channel tile
    int wgrp;     // group of NPH consecutive w-phases
    int pg;       // (rho_d, rho_h) phase group from the grid (unused with the phase-group loop)
    int n, grp;   // sample, channel group
};

// a / d and a % d for a wave-uniform d > 0; d == 1, the usual case for the
// channel-group, co-tile and w-phase-group counts, needs no division
CONVT3D_IX void divmod_uniform(int a, int d, int &q, int &r) {
    if (d == 1) {
        q = a;
        r = 0;
        return;
    }
    q = a / d;
    r = a - q * d;
}

CONVT3D_IX WorkItem work_item(const ConvParams &P, int bid, int gx, int gy, int gz) {
    const int total = gx * gy * gz;
    constexpr int nx = kNumXcd;
    const int q = total / nx, r = total % nx;
    const int xcd = bid % nx, idx = bid / nx;
    const int lin = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
    int bx, by;
    if (P.order == 0) {
        by = lin % gy;
        bx = (lin / gy) % gx;
    } else {
        bx = lin % gx;
        by = (lin / gx) % gy;
    }
    const int nz = lin / (gx * gy);  // grid z = sample * G + group
    WorkItem w;
    w.bx = bx;
    divmod_uniform(nz, P.G, w.n, w.grp);
    divmod_uniform(by, P.co_tiles, by, w.co_tile);
    divmod_uniform(by, P.nwgroups, w.pg, w.wgrp);
    return w;
}

// ---- tile: the region holding tile bx, then the tile's box inside it
struct TileBox {
    int reg;
    int TQd, TQh, TQw;        // box (stride-phase positions)
    int q0d, q0h, q0w;        // first position
    int TQd_e, TQh_e, TQw_e;  // extent inside the region (the box may overhang its end)
};

CONVT3D_IX TileBox tile_box(const ConvParams &P, int bx) {
    int reg = 0;
    while (reg + 1 < P.nreg && bx >= P.rg_off[reg + 1]) ++reg;
    const int *RG = P.rg[reg];
    const int local = bx - P.rg_off[reg];
    const int tw_i = local % RG[11];
    const int th_i = (local / RG[11]) % RG[10];
    const int td_i = local / (RG[11] * RG[10]);
    TileBox t;
    t.reg = reg;
    t.TQd = RG[6];
    t.TQh = RG[7];
    t.TQw = RG[8];
    t.q0d = RG[0] + td_i * t.TQd;
    t.q0h = RG[1] + th_i * t.TQh;
    t.q0w = RG[2] + tw_i * t.TQw;
    t.TQd_e = imin(t.TQd, RG[3] - t.q0d);
    t.TQh_e = imin(t.TQh, RG[4] - t.q0h);
    t.TQw_e = imin(t.TQw, RG[5] - t.q0w);
    return t;
}

// ---- input halo along d and h of the (rho_d, rho_h) groups [pg0, pg0 + npg)
// for a box of TQd x TQh positions: inputs q + c - e*j of every group's taps,
// relative to the box's first position.  A dim no tap reaches keeps the box.
CONVT3D_IX void halo_dh(const ConvParams &P, int pg0, int npg, int TQd, int TQh, int &lo_d_rel, int &HD,
                        int &lo_h_rel, int &HH) {
    const int sh = P.s3[1], ed = P.pe[0], eh = P.pe[1];
    int dlo = INT_MAX, dhi = INT_MIN, hlo = INT_MAX, hhi = INT_MIN;
    for (int g = pg0; g < pg0 + npg; ++g) {
        const int rd = g / sh, rh = g % sh;
        const int Jd_ = P.pJ[0][rd], cd_ = P.pc[0][rd], Jh_ = P.pJ[1][rh], ch_ = P.pc[1][rh];
        if (Jd_ > 0) {
            dlo = imin(dlo, cd_ - ed * (Jd_ - 1));
            dhi = imax(dhi, TQd - 1 + cd_);
        }
        if (Jh_ > 0) {
            hlo = imin(hlo, ch_ - eh * (Jh_ - 1));
            hhi = imax(hhi, TQh - 1 + ch_);
        }
    }
    lo_d_rel = 0;
    HD = TQd;
    lo_h_rel = 0;
    HH = TQh;
    if (dlo <= dhi) {
        lo_d_rel = dlo;
        HD = dhi - dlo + 1;
    }
    if (hlo <= hhi) {
        lo_h_rel = hlo;
        HH = hhi - hlo + 1;
    }
}

// ---- w-phase rw: its taps Jw and input offset cw; widens the halo's w range
// [lo_w_rel, hi_w_rel] (relative to the box of TQw positions; start from
// INT_MAX, INT_MIN: empty while no phase has a tap) by the inputs it reads
CONVT3D_IX void w_phase(const ConvParams &P, int rw, int TQw, int &Jw, int &cw, int &lo_w_rel, int &hi_w_rel) {
    Jw = P.pJ[2][rw];
    cw = P.pc[2][rw];
    if (Jw > 0) {
        lo_w_rel = imin(lo_w_rel, cw - P.pe[2] * (Jw - 1));
        hi_w_rel = imax(hi_w_rel, TQw - 1 + cw);
    }
}

// After the w_phase calls: true when some phase has a tap.  Otherwise the
// halo's w range is set to the box itself (no tap reads it; this keeps the
// halo origin q0w + lo_w_rel finite).
CONVT3D_IX bool w_halo_close(int TQw, int &lo_w_rel, int &hi_w_rel) {
    if (lo_w_rel <= hi_w_rel) return true;
    lo_w_rel = 0;
    hi_w_rel = TQw - 1;
    return false;
}

// ---- tap index range [lo, hi] of a phase (input offset c, step e, J taps)
// that reaches the input [0, in) from some position of [q0, q0 + te - 1]
CONVT3D_IX void tap_range(int q0, int te, int c, int e, int J, int in, int &lo, int &hi) {
    lo = imax(0, ceil_div_any(q0 + c - (in - 1), e));
    hi = imin(J - 1, floor_div_any(q0 + te - 1 + c, e));
}

// ---- column c of position block blk (32 columns each) of the box (d
// slowest, w fastest) -> position; true when the position is inside the
// tile's extent (a column past the box volume decodes as position 0)
CONVT3D_IX bool pos_decode(int blk, int c, int vol, int plane, int TQw, int TQd_e, int TQh_e, int TQw_e, int &td,
                           int &th, int &tw) {
    const int pidx = blk * 32 + c;
    const int pi = pidx < vol ? pidx : 0;
    td = pi / plane;
    const int rem = pi - td * plane;
    th = rem / TQw;
    tw = rem - th * TQw;
    return pidx < vol && td < TQd_e && th < TQh_e && tw < TQw_e;
}

// ---- LDS layout of a staged chunk: float4 [octet][k-row h][d][h][w]; a slab
// is HD*HH*HW positions.  float4 index of the B operands of a lane (k-row
// `half`) at tap offset 0, and of a group (taps jd, jh, jw; octet g4 of the
// chunk) relative to it.
CONVT3D_IX int b_lane_off(int half, int SLAB, int td, int th, int tw, int HH, int HW) {
    return half * SLAB + (td * HH + th) * HW + tw;
}
CONVT3D_IX int b_group_off(int cd, int ed, int jd, int lo_d_rel, int ch, int eh, int jh, int lo_h_rel, int cw,
                           int ew, int jw, int lo_w_rel, int HH, int HW, int g4, int slab2) {
    return ((cd - ed * jd - lo_d_rel) * HH + (ch - eh * jh - lo_h_rel)) * HW + (cw - ew * jw - lo_w_rel) + g4 * slab2;
}
// float4 index of halo position pos of octet g (channel pair half) in a chunk
CONVT3D_IX int stage_lds_index(int g, int SLAB, int pos, int half) { return (2 * g + half) * SLAB + pos; }

// ---- packed weights: float4 index of group (octet g4 of chunk, taps jd, jh,
// jw) of lane 0 within a co block of a phase (ntp taps, Jh x jwn sub-kernel)
CONVT3D_IX int a_group_index(int chunk, int G4, int g4, int ntp, int jd, int Jh, int jh, int jwn, int jw) {
    return ((chunk * G4 + g4) * ntp + (jd * Jh + jh) * jwn + jw) * 64;
}
// float4 index of a co block's first group of phase ph
CONVT3D_IX int a_block_base(const ConvParams &P, int ph, int cb) { return (P.wp_off[ph] >> 2) + cb * P.steps4[ph] * 64; }

// ---- outputs: element offset of voxel (od, oh, ow) of the lane's row pair
// (k-row half: 4 channels further) from its row base
CONVT3D_IX int out_voxel_off(int half, int S, int od, int Ho, int oh, int Wo, int ow) {
    return 4 * half * S + (od * Ho + oh) * Wo + ow;
}
// accumulator row of co block c, register r: output channel row0 + this (+ 4*half)
CONVT3D_IX int acc_row(int row0, int c, int r) { return row0 + c * 32 + 8 * (r >> 2) + (r & 3); }

// bytes from the base of accumulator row `row` (channel row; its upper
// k-row half writes the channel 4 further, at 4*S floats) that belong to
// existing channels: both rows, the lower one only, or none.  A buffer
// descriptor of this range drops the stores of the other lanes.
CONVT3D_IX unsigned row_pair_bytes(int row, int Cout, int S) {
    return row + 4 < Cout ? 20u * (unsigned)S : row < Cout ? 4u * (unsigned)S : 0u;
}
// byte offset a lane gives a store that must not happen: past every range
constexpr unsigned kDropOffset = 0xFFFFFFF8u;

// ---- halo staging: raw buffer loads of one channel chunk (CI_T channel
// planes from the chunk's first channel, CI_T * D*H*W * 4 bytes, the plane
// offset of each channel in the scalar offset), or, when that range passes
// 2^31 bytes, of one channel plane per descriptor (range 4 * D*H*W, no scalar
// offset).  A halo position outside the input gets this byte offset, past
// either range whether or not the scalar offset is added before the range
// check, and reads as zero.  The planner keeps D*H*W at or below 2^29, so both
// ranges stay at or below 2^31 bytes and the offset plus a plane offset below
// 2^32.
constexpr unsigned kHaloOutside = 0x80000000u;
static_assert(kMaxChunkPlanes <= (int64_t(1) << 29) && kMaxInputPlane <= (int64_t(1) << 29),
              "staging ranges and the outside offset must fit 32 bits");
// a 64-bit address from its two 32-bit halves (each read from the first
// lane into a scalar register), both zero-extended
CONVT3D_IX uint64_t join_halves(unsigned hi, unsigned lo) { return ((uint64_t)hi << 32) | (uint64_t)lo; }
// range of the chunk descriptor (0: one descriptor per plane instead)
CONVT3D_IX unsigned chunk_range_bytes(int CI_T, int DHWin) { return 4u * (unsigned)CI_T * (unsigned)DHWin; }
// byte offset of halo position (id, ih, iw) in a channel plane, or kHaloOutside
CONVT3D_IX unsigned halo_src_off(int id, int ih, int iw, int D, int H, int W) {
    const bool inside = (unsigned)id < (unsigned)D && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
    return inside ? (unsigned)((id * H + ih) * W + iw) * 4u : kHaloOutside;
}

// ---- statistics partials, channel-major [n][Cout_total][tile][2] (each
// channel's tiles contiguous, the order the statistics merges read them):
// tile index of a work item, and the float offset of a (sum, sum of squares)
CONVT3D_IX int partial_tile(const ConvParams &P, int rho_d, int rho_h, int wgrp, int bx) {
    return ((rho_d * P.s3[1] + rho_h) * P.nwgroups + wgrp) * P.tiles_total + bx;
}
CONVT3D_IX size_t partial_offset(int n, int C_total, int c, int tiles, int tile) {
    return (((size_t)n * C_total + c) * tiles + tile) * 2;
}

}  // namespace ix
}  // namespace convt3d
