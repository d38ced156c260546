// Host replay of libconvt3d's kernel address arithmetic (test infrastructure).
//
// The library's C ABI (api.cpp) and planner (plan.cpp) are linked as they
// are; the launch_* functions that would enqueue HIP kernels are replaced by
// CPU replays that walk every workgroup, wave and lane of the launch and check
// each address the kernel would form -- through the same index functions the
// convolution kernel calls (conv_index.hpp) -- against the buffers the caller
// handed in: LDS inside the workgroup's dynamic allocation (and never read
// before it was staged), global reads inside x / the packed
// weights / bias / the partials, every output and partial sum written exactly
// once, and the statistics merges reading only partials the conv wrote.
// No value is computed.  Built with -fsanitize=address,undefined, so the host
// code of the planner and the C ABI runs under the sanitizers too.
//
// Input: one case per line on stdin,
//   name n cin cout d h w  kd kh kw  sd sh sw  pd ph pw  od oh ow  dd dh dw
//   groups epi gn_groups plan_env phase_loop_env mode
// plan_env / phase_loop_env: value of CONVT3D_PLAN / CONVT3D_PHASE_LOOP or
// "-" for unset.  mode: "full" (the plan convt3d_fused runs, checked lane by
// lane with LDS validity and output coverage; then every other plan
// convt3d_autotune may time -- both of its stages -- by address ranges),
// "fast" (all of them by address ranges) or "one" (only the plan
// convt3d_fused runs, by address ranges: full-size tensors).  Output: one
// line per case, "ok ..." or "FAIL ..."; exit status 1 if any case failed.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cinttypes>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <memory>
#include <string>
#include <thread>
#include <vector>

#include "conv_index.hpp"
#include "convt3d.h"
#include "convt3d_internal.hpp"

using namespace convt3d;

// ---------------------------------------------------------------------------
// HIP runtime entry points the C ABI references (events are only used for
// timing and tuning, which the replay never asks for).
extern "C" {
hipError_t hipEventCreate(hipEvent_t *e) {
    if (e) *e = nullptr;
    return hipErrorNotSupported;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipErrorNotSupported; }
hipError_t hipEventElapsedTime(float *, hipEvent_t, hipEvent_t) { return hipErrorNotSupported; }
}

namespace {

// ---------------------------------------------------------------------------
// registered "device" buffers (host memory standing in for them)
struct Buf {
    std::string name;
    char *base = nullptr;
    size_t bytes = 0;
    std::vector<uint8_t> writes;  // per float: times written (coverage), when tracked
};
std::vector<std::unique_ptr<Buf>> g_bufs;
bool g_full = true;
int g_errors = 0;
long long g_checks = 0;
std::string g_first_error;

void fail(const char *fmt, ...) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    if (g_errors++ == 0) g_first_error = msg;
}

Buf *new_buf(const char *name, size_t bytes, bool track) {
    auto b = std::make_unique<Buf>();
    b->name = name;
    b->bytes = bytes;
    const size_t alloc = ((bytes + 255) / 256 + 1) * 256;
    b->base = static_cast<char *>(std::aligned_alloc(256, alloc));
    if (track) b->writes.assign(bytes / 4 + 1, 0);
    g_bufs.push_back(std::move(b));
    return g_bufs.back().get();
}
void free_bufs() {
    for (auto &b : g_bufs) std::free(b->base);
    g_bufs.clear();
}
Buf *find_buf(const void *p) {
    const char *c = static_cast<const char *>(p);
    for (auto &b : g_bufs)
        if (c >= b->base && c < b->base + std::max<size_t>(b->bytes, 1)) return b.get();
    return nullptr;
}

// [base + off_floats, + n_floats) inside buffer b; optional write / read-written tracking
bool in_buf(const Buf *b, const float *base, int64_t off_floats, int64_t n_floats, const char *what) {
    ++g_checks;
    const char *p = reinterpret_cast<const char *>(base) + off_floats * 4;
    if (!b || off_floats < 0 || p < b->base || p + n_floats * 4 > b->base + b->bytes) {
        fail("%s: float offset %" PRId64 " (+%" PRId64 ") outside %s (%zu bytes)", what, off_floats, n_floats,
             b ? b->name.c_str() : "no buffer", b ? b->bytes : (size_t)0);
        return false;
    }
    return true;
}
void mark_write(Buf *b, const float *base, int64_t off, const char *what) {
    if (!in_buf(b, base, off, 1, what) || b->writes.empty()) return;
    const size_t i = (reinterpret_cast<const char *>(base + off) - b->base) / 4;
    if (b->writes[i] == 255) return;
    if (++b->writes[i] > 1) fail("%s: float %zu of %s written twice", what, i, b->name.c_str());
}
void check_written(Buf *b, const float *base, int64_t off, const char *what) {
    if (!in_buf(b, base, off, 1, what) || b->writes.empty()) return;
    const size_t i = (reinterpret_cast<const char *>(base + off) - b->base) / 4;
    if (b->writes[i] == 0) fail("%s: float %zu of %s read but never written", what, i, b->name.c_str());
}

// ---------------------------------------------------------------------------
// convolution kernel replay
int replay_conv(const Plan &pl, const ConvParams &P) {
    const Variant v = kVariants[pl.variant];
    const int CBW = v.CBW, NPH = v.NPH, PBW = v.PBW;
    const bool SM = v.softmax, PL = pl.phase_loop != 0;
    if (PL && !v.phase_loop) fail("variant %d has no phase-loop build", pl.variant);
    if (pl.lds_bytes > kMaxLdsBytes) fail("LDS %d bytes over the %d limit", pl.lds_bytes, kMaxLdsBytes);
    const int gx = (int)pl.grid_x, gy = (int)pl.grid_y, gz = (int)pl.grid_z;
    if (gx < 1 || gy < 1 || gz < 1 || gy > 65535 || gz > 65535) fail("grid %d x %d x %d", gx, gy, gz);
    if (gx != P.tiles_total) fail("grid x %d != tiles %d", gx, P.tiles_total);
    const int lds_floats = pl.lds_bytes / 4;
    const int CO_T = P.WCO * CBW, CO32 = CO_T * 32;
    if (P.WCO * P.WPOS != 4) fail("wave grid %d x %d", P.WCO, P.WPOS);
    if (P.red_off + P.WPOS * CO32 * 2 > lds_floats)
        fail("reduction scratch [%d, %d) past LDS %d floats", P.red_off, P.red_off + P.WPOS * CO32 * 2, lds_floats);
    Buf *bx_ = find_buf(P.x), *bw = find_buf(P.wp), *bo = find_buf(P.out);
    Buf *bp = P.partials ? find_buf(P.partials) : nullptr;
    Buf *bb = P.bias ? find_buf(P.bias) : nullptr;
    const int sd = P.s3[0], sh = P.s3[1], sw = P.s3[2];
    const int ed = P.pe[0], eh = P.pe[1], ew = P.pe[2];
    const int DHWin = P.D * P.H * P.W;
    const int S = P.Do * P.Ho * P.Wo;
    const bool gn = P.epi == CONVT3D_EPI_RELU_GROUPNORM, bn = P.epi == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL;
    const bool stores = !bn;  // the pooled BatchNorm kernel never writes out
    if ((gn || bn) && !bp) fail("statistics epilogue without partials");
    if (sw % NPH) fail("NPH %d does not divide stride %d", NPH, sw);
    if (P.nwgroups * NPH != sw) fail("w-phase groups %d x NPH %d != stride %d", P.nwgroups, NPH, sw);
    if (gy != P.co_tiles * (PL ? 1 : sd * sh) * P.nwgroups) fail("grid y %d", gy);
    if (P.CI_T % 8 || P.nchunks * P.CI_T < P.octets * 8 || (P.nchunks - 1) * P.CI_T >= P.octets * 8)
        fail("channel chunks %d x %d for %d octets", P.nchunks, P.CI_T, P.octets);
    if (PL && P.nchunks != 1) fail("phase-group loop with %d channel chunks", P.nchunks);
    const int G4 = P.CI_T >> 3;
    std::vector<uint8_t> ldsv;  // LDS float4 validity (full mode)

    for (int bid = 0; bid < gx * gy * gz; ++bid) {
        const ix::WorkItem wi = ix::work_item(P, bid, gx, gy, gz);
        const int n = wi.n, grp = wi.grp;
        if (n < 0 || n >= P.N || grp < 0 || grp >= P.G || wi.bx < 0 || wi.bx >= gx || wi.co_tile >= P.co_tiles ||
            wi.wgrp >= P.nwgroups || (!PL && wi.pg >= sd * sh)) {
            fail("workgroup %d decodes to n %d grp %d tile %d co %d wg %d pg %d", bid, n, grp, wi.bx, wi.co_tile,
                 wi.wgrp, wi.pg);
            continue;
        }
        const ix::TileBox tb = ix::tile_box(P, wi.bx);
        if (tb.TQd_e < 1 || tb.TQh_e < 1 || tb.TQw_e < 1) fail("tile %d is empty", wi.bx);
        const int TQd = tb.TQd, TQh = tb.TQh, TQw = tb.TQw;
        const int npg = PL ? sd * sh : 1, pg0 = PL ? 0 : wi.pg;
        int lo_d_rel, HD, lo_h_rel, HH;
        ix::halo_dh(P, pg0, npg, TQd, TQh, lo_d_rel, HD, lo_h_rel, HH);
        int Jw[2] = {0, 0}, cw[2] = {0, 0}, rw[2] = {0, 0};
        int lo_w_rel = INT_MAX, hi_w_rel = INT_MIN;
        for (int p = 0; p < NPH; ++p) {
            rw[p] = wi.wgrp * NPH + p;
            ix::w_phase(P, rw[p], TQw, Jw[p], cw[p], lo_w_rel, hi_w_rel);
        }
        const bool w_taps = ix::w_halo_close(TQw, lo_w_rel, hi_w_rel);
        const int HW = hi_w_rel - lo_w_rel + 1;
        const int lo_d = tb.q0d + lo_d_rel, lo_h = tb.q0h + lo_h_rel, lo_w = tb.q0w + lo_w_rel;
        int jw_lo[2], jw_hi[2];
        for (int p = 0; p < NPH; ++p) ix::tap_range(tb.q0w, tb.TQw_e, cw[p], ew, Jw[p], P.W, jw_lo[p], jw_hi[p]);
        const int SLAB = HD * HH * HW, slab2 = 2 * SLAB;
        // a register-prefetch kernel stages every later chunk from kRpPositions
        // positions per thread: the halo must fit them, one octet per chunk
        if (v.prefetch && (SLAB > kRpPositions * kBlockThreads || P.CI_T != kOctet || P.plane_desc || PL))
            fail("prefetch kernel: halo of %d positions, chunk %d, plane descriptors %d", SLAB, P.CI_T, P.plane_desc);
        const int halo4 = (P.CI_T * SLAB) >> 2;  // float4s of the staged chunk
        if (halo4 * 4 > P.red_off) fail("halo of %d floats overlaps the reduction scratch at %d", halo4 * 4, P.red_off);
        const int vol = TQd * TQh * TQw, plane = TQh * TQw;
        if (vol > P.WPOS * PBW * 32) fail("box volume %d over the %d columns of the workgroup", vol, P.WPOS * PBW * 32);
        const int cb0w = wi.co_tile * CO_T;
        if (g_full) ldsv.assign(lds_floats / 4 + 1, 0);

        const int inc_w = kBlockThreads % HW, inc_h = (kBlockThreads / HW) % HH, inc_d = kBlockThreads / (HW * HH);
        const unsigned plane_bytes = 4u * (unsigned)DHWin;
        if ((int64_t)DHWin > kMaxInputPlane) fail("input plane of %d voxels", DHWin);
        if (P.plane_desc != ((int64_t)P.CI_T * DHWin > kMaxChunkPlanes))
            fail("plane descriptors %d for a chunk of %d planes of %d", P.plane_desc, P.CI_T, DHWin);
        // one descriptor over the chunk (scalar offset: the channel's plane) or one per plane
        const uint64_t range = P.plane_desc ? plane_bytes : ix::chunk_range_bytes(P.CI_T, DHWin);
        if (range > (uint64_t(1) << 31)) fail("staging range %" PRIu64 " bytes", range);
        auto stage = [&](int chunk) {
            const int oct0 = chunk * G4;
            for (int t = 0; t < kBlockThreads; ++t) {
                int w = t % HW, h = (t / HW) % HH, d = t / (HW * HH);
                for (int pos = t; pos < SLAB; pos += kBlockThreads) {
                    if ((d * HH + h) * HW + w != pos) fail("staging digits (%d,%d,%d) != position %d", d, h, w, pos);
                    const int id = lo_d + d, ih = lo_h + h, iw = lo_w + w;
                    const bool inside =
                        (unsigned)id < (unsigned)P.D && (unsigned)ih < (unsigned)P.H && (unsigned)iw < (unsigned)P.W;
                    const unsigned vo = ix::halo_src_off(id, ih, iw, P.D, P.H, P.W);
                    for (int g = 0; g < G4; ++g) {
                        const int ci0 = (oct0 + g) * 8;
                        const int nch = std::min(8, P.Cin - ci0);  // channels loaded
                        for (int c = 0; c < nch; ++c) {
                            const int ch = 8 * g + c;  // channel of the chunk
                            // descriptor base (floats from the chunk's first plane)
                            // and the load's buffer offset: in the range exactly
                            // when the position is inside the input, with or
                            // without the scalar offset, and never wrapping
                            const int64_t base = P.plane_desc ? (int64_t)ch * DHWin : 0;
                            const uint64_t so = P.plane_desc ? 0u : (uint64_t)ch * plane_bytes;
                            const uint64_t vso = (uint64_t)vo + so;
                            if (vso >= (uint64_t(1) << 32)) fail("staging offset %" PRIu64 " wraps", vso);
                            if (inside != (vso < range) || inside != (vo < range))
                                fail("staging offset %" PRIu64 " (position %s) against range %" PRIu64, vso,
                                     inside ? "inside" : "outside", range);
                            if (inside && (g_full || pos == t || pos + kBlockThreads >= SLAB)) {
                                const int64_t rel = base + (int64_t)(vso / 4);  // floats from the chunk's first plane
                                const int64_t off = (int64_t)n * P.x_nstride + (int64_t)grp * P.xg +
                                                    (int64_t)oct0 * 8 * DHWin + rel;
                                if (c == 0 || c == nch - 1) in_buf(bx_, P.x, off, 1, "x read");
                                if (rel != (int64_t)(ci0 - oct0 * 8 + c) * DHWin + (vo / 4))
                                    fail("staging offset %" PRIu64 " is not channel %d's", vso, ci0 + c);
                            }
                        }
                        for (int half = 0; half < 2; ++half) {
                            const int li = ix::stage_lds_index(g, SLAB, pos, half);
                            if (li < 0 || li >= halo4) fail("staging LDS float4 %d outside the halo (%d)", li, halo4);
                            else if (g_full) ldsv[li] = 1;
                        }
                    }
                    w += inc_w;
                    if (w >= HW) { w -= HW; ++h; }
                    h += inc_h;
                    if (h >= HH) { h -= HH; ++d; }
                    d += inc_d;
                }
            }
        };
        stage(0);

        for (int pgi = 0; pgi < npg; ++pgi) {
            const int pg = pg0 + pgi;
            const int rho_h = pg % sh, rho_d = pg / sh;
            const int Jd = P.pJ[0][rho_d], cd = P.pc[0][rho_d], Jh = P.pJ[1][rho_h], ch = P.pc[1][rho_h];
            int jd_lo, jd_hi, jh_lo, jh_hi;
            ix::tap_range(tb.q0d, tb.TQd_e, cd, ed, Jd, P.D, jd_lo, jd_hi);
            ix::tap_range(tb.q0h, tb.TQh_e, ch, eh, Jh, P.H, jh_lo, jh_hi);
            bool work = Jd > 0 && Jh > 0 && w_taps && jd_lo <= jd_hi && jh_lo <= jh_hi;
            bool anyw = false;
            for (int p = 0; p < NPH; ++p) anyw = anyw || (Jw[p] > 0 && jw_lo[p] <= jw_hi[p]);
            work = work && anyw;
            if (work) {
                for (int chunk = 0; chunk < P.nchunks; ++chunk) {
                    if (!PL && chunk > 0) stage(chunk);
                    for (int p = 0; p < NPH; ++p) {
                        if (Jw[p] == 0 || jw_lo[p] > jw_hi[p]) continue;
                        const int ph = (rho_d * sh + rho_h) * sw + rw[p];
                        const int ntp = P.ntaps[ph];
                        if (ntp != Jd * Jh * Jw[p]) fail("phase %d: %d taps, expected %d", ph, ntp, Jd * Jh * Jw[p]);
                        if (P.steps4[ph] != P.octets * ntp) fail("phase %d: steps4", ph);
                        const int n_it = (jd_hi - jd_lo + 1) * (jh_hi - jh_lo + 1) * (jw_hi[p] - jw_lo[p] + 1) * G4;
                        for (int wave = 0; wave < 4; ++wave) {
                            const int wco = wave % P.WCO, wpos = wave / P.WCO;
                            const bool wave_live = std::min(vol, tb.TQd_e * plane) > wpos * PBW * 32;
                            if (!wave_live) continue;
                            const int cb0 = cb0w + wco * CBW;
                            // the lanes' B offsets at tap offset 0
                            std::vector<int> loff(64 * PBW);
                            int lmin = INT_MAX, lmax = INT_MIN;
                            for (int lane = 0; lane < 64; ++lane)
                                for (int pb = 0; pb < PBW; ++pb) {
                                    int td, th, tw;
                                    ix::pos_decode(wpos * PBW + pb, lane & 31, vol, plane, TQw, tb.TQd_e, tb.TQh_e,
                                                   tb.TQw_e, td, th, tw);
                                    const int o = ix::b_lane_off(lane >> 5, SLAB, td, th, tw, HH, HW);
                                    loff[lane * PBW + pb] = o;
                                    lmin = std::min(lmin, o);
                                    lmax = std::max(lmax, o);
                                }
                            int jd = jd_lo, jh = jh_lo, jw = jw_lo[p], g4 = 0;
                            for (int it = 0; it < n_it; ++it) {
                                const int gi = ix::a_group_index(chunk, G4, g4, ntp, jd, Jh, jh, Jw[p], jw);
                                const int bo2 = ix::b_group_off(cd, ed, jd, lo_d_rel, ch, eh, jh, lo_h_rel, cw[p], ew,
                                                                jw, lo_w_rel, HH, HW, g4, slab2);
                                // A operands: float4 gi + lane of each co block's phase block
                                if (gi < 0 || gi + 64 > P.steps4[ph] * 64)
                                    fail("A group %d outside the phase block (%d float4)", gi, P.steps4[ph] * 64);
                                for (int c = 0; c < CBW; ++c) {
                                    const int cb = std::min(cb0 + c, P.cb_total - 1);
                                    const int64_t f4 = ix::a_block_base(P, ph, cb) + gi;
                                    in_buf(bw, P.wp, (int64_t)grp * P.wpg + f4 * 4, 64 * 4, "A operand read");
                                    if (f4 * 4 + 256 > P.wpg) fail("A operand read past the group's packed weights");
                                }
                                // B operands
                                if (bo2 + lmin < 0 || bo2 + lmax >= halo4)
                                    fail("B read float4 [%d, %d] outside the halo (%d) (tile %d, pg %d, chunk %d)",
                                         bo2 + lmin, bo2 + lmax, halo4, wi.bx, pg, chunk);
                                else if (g_full)
                                    for (int i = 0; i < 64 * PBW; ++i)
                                        if (!ldsv[loff[i] + bo2]) {
                                            fail("B read of LDS float4 %d before it was written (tile %d)",
                                                 loff[i] + bo2, wi.bx);
                                            break;
                                        }
                                ++g_checks;
                                if (++g4 == G4) {
                                    g4 = 0;
                                    if (++jw > jw_hi[p]) {
                                        jw = jw_lo[p];
                                        if (++jh > jh_hi) { jh = jh_lo; ++jd; }
                                    }
                                }
                            }
                            if (jd != jd_hi + 1 && n_it > 0) fail("group iteration ended at jd %d", jd);
                        }
                    }
                }
            }

            // ---- epilogue
            const int Cout = P.Cout;
            const bool blk8 = gn && P.gn_block8;
            for (int wave = 0; wave < 4; ++wave) {
                const int wco = wave % P.WCO, wpos = wave / P.WCO;
                const int row0 = (cb0w + wco * CBW) * 32;
                const bool rows_full = row0 + CBW * 32 <= Cout;
                const int64_t rowbase = (int64_t)n * P.Cout_total + (int64_t)grp * Cout;
                for (int lane = 0; lane < 64; ++lane) {
                    const int half = lane >> 5, col = lane & 31;
                    auto row_ok = [&](int c, int r) { return rows_full || ix::acc_row(row0, c, r) + 4 * half < Cout; };
                    for (int pb = 0; pb < PBW; ++pb) {
                        int td, th, tw;
                        const bool pos_ok = ix::pos_decode(wpos * PBW + pb, col, vol, plane, TQw, tb.TQd_e, tb.TQh_e,
                                                           tb.TQw_e, td, th, tw);
                        const int od = sd * (tb.q0d + td) + rho_d, oh = sh * (tb.q0h + th) + rho_h;
                        bool okp[2];
                        int vofs[2];
                        for (int p = 0; p < NPH; ++p) {
                            const int ow = sw * (tb.q0w + tw) + rw[p];
                            okp[p] = pos_ok && od < P.Do && oh < P.Ho && ow < P.Wo;
                            vofs[p] = ix::out_voxel_off(half, S, od, P.Ho, oh, P.Wo, ow);
                            if (okp[p] && (int64_t)vofs[p] * 4 >= (int64_t(1) << 32)) fail("byte offset past 2^32");
                        }
                        const bool pair = NPH == 2 && okp[0] && okp[1] && P.Wo % 2 == 0;
                        if (pair && (vofs[0] & 1)) fail("float pair store not 8-byte aligned");
                        if (!stores) continue;
                        if (!g_full && !(lane == 0 || lane == 31 || lane == 32 || lane == 63)) continue;
                        for (int c = 0; c < CBW; ++c)
                            for (int r = 0; r < 16; ++r) {
                                const int row = ix::acc_row(row0, c, r);
                                // the softmax kernels store through a buffer descriptor per row that
                                // drops stores past the row pair's existing channels; the others branch
                                const bool cok = SM ? true : blk8 ? row_ok(c, 4 * (r >> 2)) : row_ok(c, r);
                                if (!cok) continue;
                                if (P.bias && row_ok(c, r))
                                    in_buf(bb, P.bias, (int64_t)grp * Cout + row + 4 * half, 1, "bias read");
                                const int64_t base = (rowbase + row) * S;
                                for (int p = 0; p < NPH; ++p)
                                    if (okp[p]) {
                                        // a float pair is one store at the first phase's offset
                                        const uint64_t end = pair ? (uint64_t)vofs[0] * 4 + 8 : (uint64_t)vofs[p] * 4 + 4;
                                        if (SM && end > ix::row_pair_bytes(row, Cout, S))
                                            continue;  // dropped by the descriptor's range
                                        if (g_full) mark_write(bo, P.out, base + vofs[p], "output store");
                                        else in_buf(bo, P.out, base + vofs[p], 1, "output store");
                                    }
                            }
                    }
                }
                // statistics: LDS reduction scratch, then the tile partials
                if (gn || bn) {
                    for (int c = 0; c < CBW; ++c)
                        for (int rr = 0; rr < 32; ++rr) {
                            const int row = (wco * CBW + c) * 32 + rr;
                            const int ri = P.red_off + (wpos * CO32 + row) * 2 + 1;
                            if (ri >= lds_floats || ri < halo4 * 4) fail("reduction scratch float %d outside", ri);
                        }
                }
            }
            if (gn || bn) {
                const int tile = ix::partial_tile(P, rho_d, rho_h, wi.wgrp, wi.bx);
                if (tile < 0 || tile >= P.tiles_per_n) fail("partial tile %d of %d", tile, P.tiles_per_n);
                for (int row = 0; row < CO32; ++row) {
                    const int co = wi.co_tile * CO32 + row;
                    if (co >= Cout) continue;
                    if (blk8 && (row & 7) != 0) continue;
                    const int64_t pi = (int64_t)ix::partial_offset(n, P.Cout_total, grp * Cout + co, P.tiles_per_n, tile);
                    mark_write(bp, P.partials, pi, "partial store");
                    mark_write(bp, P.partials, pi + 1, "partial store");
                }
            }
        }
    }
    return 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers of the library, replayed
namespace convt3d {

int launch_prepack(const Plan &pl, const float *w, float *wp, void *) {
    Buf *bw = find_buf(w), *bp = find_buf(wp);
    const int64_t slice = (int64_t)pl.cig * pl.cog * pl.g.k[0] * pl.g.k[1] * pl.g.k[2];
    in_buf(bw, w, 0, slice, "weight slice read");
    in_buf(bp, wp, 0, pl.packed_floats, "packed weights write");
    for (int ph = 0; ph < pl.nph; ++ph) {
        const int sh = pl.s3[1], sw = pl.s3[2];
        const int rd = ph / (sh * sw), rh = (ph / sw) % sh, rw = ph % sw;
        for (int dim = 0; dim < 3; ++dim) {
            const int rr = dim == 0 ? rd : dim == 1 ? rh : rw;
            const DimPhase &d = pl.ph[dim][rr];
            if (d.J > 0 && d.r + pl.ts[dim] * (d.J - 1) >= pl.g.k[dim]) fail("phase tap past the kernel");
        }
        if (pl.wp_off[ph] + (int64_t)pl.cb_total * pl.steps4[ph] * 256 > pl.packed_floats) fail("phase block past the end");
    }
    return 0;
}

int launch_conv(const Plan &pl, const ConvParams &cp, void *) { return replay_conv(pl, cp); }

int launch_gn_finalize(const float *partials, int N, int tiles_per_n, int C, int G, int chan_step, double,
                       float, const float *gamma, const float *beta, float *ab, float *stats_out, const float *prow,
                       const float *pbias, double, void *) {
    if (prow) in_buf(find_buf(prow), prow, 0, (int64_t)N * C, "pivot read");
    if (pbias) in_buf(find_buf(pbias), pbias, 0, C, "bias pivot read");
    Buf *bp = find_buf(partials), *ba = find_buf(ab);
    const int cpg = C / G;
    if (cpg % chan_step) fail("channel step %d does not divide %d channels per group", chan_step, cpg);
    for (int n = 0; n < N; ++n)
        for (int g = 0; g < G; ++g)
            for (int t = 0; t < tiles_per_n; ++t)
                for (int cc = 0; cc < cpg; cc += chan_step) {
                    const int64_t i = (int64_t)ix::partial_offset(n, C, g * cpg + cc, tiles_per_n, t);
                    check_written(bp, partials, i, "GroupNorm partial read");
                    check_written(bp, partials, i + 1, "GroupNorm partial read");
                }
    in_buf(ba, ab, 0, (int64_t)N * C * 2, "GroupNorm scale/shift write");
    if (gamma) in_buf(find_buf(gamma), gamma, 0, C, "gamma");
    if (beta) in_buf(find_buf(beta), beta, 0, C, "beta");
    if (stats_out) in_buf(find_buf(stats_out), stats_out, 0, (int64_t)N * G * 2, "GroupNorm stats write");
    return 0;
}

int launch_normalize(const float *src, float *out, const float *ab, int rows, int64_t S, bool, void *, bool) {
    in_buf(find_buf(src), src, 0, (int64_t)rows * S, "normalise read");
    in_buf(find_buf(out), out, 0, (int64_t)rows * S, "normalise write");
    in_buf(find_buf(ab), ab, 0, (int64_t)rows * 2, "normalise scale/shift read");
    if (S % 4 == 0 && ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(out)) & 15))
        fail("normalise float4 access misaligned");
    return 0;
}

int launch_bn_finalize(const float *partials, int N, int tiles_per_n, int C, double, const convt3d_epilogue &e,
                       float *out, const float *prow, const float *pbias, void *) {
    if (prow) in_buf(find_buf(prow), prow, 0, (int64_t)N * C, "pivot read");
    if (pbias) in_buf(find_buf(pbias), pbias, 0, C, "bias pivot read");
    Buf *bp = find_buf(partials);
    for (int n = 0; n < N; ++n)
        for (int t = 0; t < tiles_per_n; ++t)
            for (int c = 0; c < C; ++c) {
                const int64_t i = (int64_t)ix::partial_offset(n, C, c, tiles_per_n, t);
                check_written(bp, partials, i, "BatchNorm partial read");
                check_written(bp, partials, i + 1, "BatchNorm partial read");
            }
    in_buf(find_buf(out), out, 0, (int64_t)N * C, "pooled output write");
    if (e.stats_out) in_buf(find_buf(e.stats_out), e.stats_out, 0, (int64_t)C * 2, "BatchNorm stats write");
    if (e.running_mean) in_buf(find_buf(e.running_mean), e.running_mean, 0, C, "running mean");
    if (e.running_var) in_buf(find_buf(e.running_var), e.running_var, 0, C, "running var");
    return 0;
}

int launch_row_stats(const float *y, int N, int C, int64_t S, bool, float, float *partials, float *pivots, void *) {
    in_buf(find_buf(pivots), pivots, 0, (int64_t)N * C, "pivot write");
    in_buf(find_buf(y), y, 0, (int64_t)N * C * S, "statistics pass read");
    in_buf(find_buf(partials), partials, 0, (int64_t)N * row_stat_chunks(S) * C * 2, "statistics pass write");
    return 0;
}

int launch_softmax_pass(const float *src, float *out, int N, int C, int64_t S, void *) {
    in_buf(find_buf(src), src, 0, (int64_t)N * C * S, "softmax pass read");
    in_buf(find_buf(out), out, 0, (int64_t)N * C * S, "softmax pass write");
    return 0;
}

int launch_bn_eval_rows(const float *partials, int N, int chunks, int C, double, const convt3d_epilogue &,
                        float *out, const float *pivots, void *) {
    in_buf(find_buf(pivots), pivots, 0, (int64_t)N * C, "pivot read");
    in_buf(find_buf(partials), partials, 0, (int64_t)N * chunks * C * 2, "eval rows read");
    in_buf(find_buf(out), out, 0, (int64_t)N * C, "eval rows write");
    return 0;
}

int launch_eval_pack(const EvalGeom &E, const float *w, float *wb, void *) {
    in_buf(find_buf(w), w, 0, (int64_t)E.Cin * E.cog * E.k3[0] * E.k3[1] * E.k3[2], "eval pack read");
    in_buf(find_buf(wb), wb, 0, (int64_t)E.Cout * E.cig * E.nbins, "eval pack write");
    return 0;
}

int launch_eval_binsum(const EvalGeom &E, const float *x, float *R, void *) {
    in_buf(find_buf(x), x, 0, (int64_t)E.N * E.Cin * E.D * E.H * E.W, "bin sum read");
    in_buf(find_buf(R), R, 0, (int64_t)E.N * E.Cin * E.nchunk * E.nbins, "bin sum write");
    for (int dim = 0; dim < 3; ++dim)
        if (E.cut[dim][0] != 0 || E.cut[dim][E.nb[dim]] != (dim == 0 ? E.D : dim == 1 ? E.H : E.W)) fail("bin cuts");
    return 0;
}

int launch_eval_finalize(const EvalGeom &E, const float *R, const float *wb, const float *bias,
                         const convt3d_epilogue &, float *out, void *) {
    in_buf(find_buf(R), R, 0, (int64_t)E.N * E.Cin * E.nchunk * E.nbins, "eval finalize read");
    in_buf(find_buf(wb), wb, 0, (int64_t)E.Cout * E.cig * E.nbins, "eval weights read");
    if (bias) in_buf(find_buf(bias), bias, 0, E.Cout, "bias");
    in_buf(find_buf(out), out, 0, (int64_t)E.N * E.Cout, "eval output write");
    return 0;
}

}  // namespace convt3d

// ---------------------------------------------------------------------------
// driver

static void set_env(const char *name, const char *v) {
    if (std::strcmp(v, "-") == 0) unsetenv(name);
    else setenv(name, v, 1);
}

static void reset_tracking() {
    for (auto &b : g_bufs) std::fill(b->writes.begin(), b->writes.end(), 0);
}

// every output float written exactly once (NONE / GroupNorm / softmax: the conv stores y)
static void check_coverage(Buf *out, int64_t elems) {
    if (!g_full || out->writes.empty()) return;
    for (int64_t i = 0; i < elems; ++i)
        if (out->writes[i] != 1) {
            fail("output float %" PRId64 " written %d times", i, (int)out->writes[i]);
            return;
        }
}

// "threads" mode: the host calls that plan (plan info, workspace size,
// output size) from several threads at once, every thread walking the cases
// in its own order, so each geometry is first planned by whichever thread
// gets there first; then a serial pass (cache hits) must give every thread's
// results.  Built with -fsanitize=thread, this checks the plan cache for data
// races.
struct PlanResult {
    int st;
    convt3d_plan_info info;
    size_t ws;
    int64_t oelems;
    bool operator==(const PlanResult &o) const {
        return st == o.st && ws == o.ws && oelems == o.oelems &&
               std::memcmp(&info, &o.info, sizeof(info)) == 0;
    }
};

static PlanResult plan_once(const convt3d_geom &g, const convt3d_epilogue &e) {
    PlanResult r;
    std::memset(&r, 0, sizeof(r));
    r.st = convt3d_get_plan_info(&g, &e, &r.info);
    r.ws = convt3d_workspace_size(&g, &e);
    r.oelems = convt3d_output_elems(&g, &e);
    return r;
}

static int threads_main(int nthreads) {
    std::vector<std::pair<convt3d_geom, convt3d_epilogue>> cases;
    char line[1024];
    while (std::fgets(line, sizeof line, stdin)) {
        if (line[0] == '#' || line[0] == '\n') continue;
        char name[128], penv[128], lenv[32], mode[16];
        convt3d_geom g{};
        int epi_kind, gn_groups;
        const int got = std::sscanf(line,
                                    "%127s %d %d %d %d %d %d  %d %d %d  %d %d %d  %d %d %d  %d %d %d  %d %d %d  %d %d %d "
                                    "%127s %31s %15s",
                                    name, &g.n, &g.cin, &g.cout, &g.d, &g.h, &g.w, &g.k[0], &g.k[1], &g.k[2], &g.stride[0],
                                    &g.stride[1], &g.stride[2], &g.pad[0], &g.pad[1], &g.pad[2], &g.out_pad[0],
                                    &g.out_pad[1], &g.out_pad[2], &g.dilation[0], &g.dilation[1], &g.dilation[2],
                                    &g.groups, &epi_kind, &gn_groups, penv, lenv, mode);
        if (got != 28) {
            std::printf("FAIL bad case line: %s", line);
            return 1;
        }
        convt3d_epilogue e{};
        e.kind = epi_kind;
        e.groups = gn_groups;
        e.eps = 1e-5f;
        e.scale = 1.0f;
        cases.emplace_back(g, e);
    }
    const int nc = (int)cases.size();
    std::vector<std::vector<PlanResult>> res(nthreads, std::vector<PlanResult>(nc));
    std::atomic<int> ready{0};
    std::vector<std::thread> pool;
    for (int t = 0; t < nthreads; ++t)
        pool.emplace_back([&, t]() {
            ready.fetch_add(1);
            while (ready.load() < nthreads) std::this_thread::yield();  // start together
            for (int i = 0; i < nc; ++i) {
                const int c = (i + t * 3) % nc;
                res[t][c] = plan_once(cases[c].first, cases[c].second);
            }
        });
    for (auto &th : pool) th.join();
    int failed = 0;
    for (int c = 0; c < nc; ++c) {
        const PlanResult want = plan_once(cases[c].first, cases[c].second);
        for (int t = 0; t < nthreads; ++t)
            if (!(res[t][c] == want)) {
                std::printf("FAIL case %d: thread %d planned status %d variant %d ws %zu, serial %d variant %d ws %zu\n",
                            c, t, res[t][c].st, res[t][c].info.variant, res[t][c].ws, want.st, want.info.variant,
                            want.ws);
                ++failed;
            }
    }
    std::printf("%d cases x %d threads, %d mismatches\n", nc, nthreads, failed);
    return failed ? 1 : 0;
}

int main(int argc, char **argv) {
    if (argc > 1 && std::strcmp(argv[1], "threads") == 0) return threads_main(argc > 2 ? std::atoi(argv[2]) : 8);
    char line[1024];
    int failed = 0, cases = 0;
    // the staging descriptor's base is rebuilt from two 32-bit halves: a low
    // half with bit 31 set must not spill into the high half
    if (ix::join_halves(0x7f12u, 0x80000004u) != 0x7f1280000004ull ||
        ix::join_halves(0u, 0xffffffffu) != 0xffffffffull) {
        std::printf("FAIL join_halves does not zero-extend\n");
        ++failed;
    }
    while (std::fgets(line, sizeof line, stdin)) {
        if (line[0] == '#' || line[0] == '\n') continue;
        char name[128], penv[128], lenv[32], mode[16];
        convt3d_geom g{};
        int epi_kind, gn_groups;
        const int got = std::sscanf(line,
                                    "%127s %d %d %d %d %d %d  %d %d %d  %d %d %d  %d %d %d  %d %d %d  %d %d %d  %d %d %d "
                                    "%127s %31s %15s",
                                    name, &g.n, &g.cin, &g.cout, &g.d, &g.h, &g.w, &g.k[0], &g.k[1], &g.k[2], &g.stride[0],
                                    &g.stride[1], &g.stride[2], &g.pad[0], &g.pad[1], &g.pad[2], &g.out_pad[0],
                                    &g.out_pad[1], &g.out_pad[2], &g.dilation[0], &g.dilation[1], &g.dilation[2],
                                    &g.groups, &epi_kind, &gn_groups, penv, lenv, mode);
        if (got != 28) {
            std::printf("FAIL bad case line: %s", line);
            ++failed;
            continue;
        }
        ++cases;
        g_full = std::strcmp(mode, "full") == 0;
        const bool candidates = std::strcmp(mode, "one") != 0;
        g_errors = 0;
        g_checks = 0;
        g_first_error.clear();
        set_env("CONVT3D_PLAN", penv);
        set_env("CONVT3D_PHASE_LOOP", lenv);
        const bool pooled = epi_kind == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL || epi_kind == CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL;

        Buf *gam = new_buf("gamma", (size_t)g.cout * 4, false);
        Buf *bet = new_buf("beta", (size_t)g.cout * 4, false);
        Buf *bias = new_buf("bias", (size_t)g.cout * 4, false);
        Buf *stats = new_buf("stats", (size_t)std::max(g.cout, g.n * std::max(gn_groups, 1)) * 2 * 4, false);
        Buf *rm = new_buf("running_mean", (size_t)g.cout * 4, false);
        Buf *rv = new_buf("running_var", (size_t)g.cout * 4, false);
        convt3d_epilogue e{};
        e.kind = epi_kind;
        e.groups = gn_groups;
        e.eps = 1e-5f;
        e.scale = 2.0f;
        e.gamma = reinterpret_cast<float *>(gam->base);
        e.beta = reinterpret_cast<float *>(bet->base);
        e.stats_out = reinterpret_cast<float *>(stats->base);
        e.momentum = 0.1f;
        if (epi_kind == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL || epi_kind == CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL) {
            e.running_mean = reinterpret_cast<float *>(rm->base);
            e.running_var = reinterpret_cast<float *>(rv->base);
        }
        convt3d_plan_info info{};
        int st = convt3d_get_plan_info(&g, &e, &info);
        if (st) {
            std::printf("FAIL %s: plan status %d\n", name, st);
            ++failed;
            free_bufs();
            continue;
        }
        const size_t ws = convt3d_workspace_size(&g, &e);
        const int64_t oelems = convt3d_output_elems(&g, &e);
        const size_t wbytes = (size_t)g.cin * (g.cout / g.groups) * g.k[0] * g.k[1] * g.k[2] * 4;
        const size_t pbytes = epi_kind == CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL ? convt3d_eval_weight_bytes(&g)
                                                                            : convt3d_packed_weight_bytes(&g);
        Buf *x = new_buf("x", (size_t)g.n * g.cin * g.d * g.h * g.w * 4, false);
        Buf *w = new_buf("w", wbytes, false);
        Buf *wp = new_buf("w_packed", pbytes, false);
        Buf *out = new_buf("out", (size_t)oelems * 4, !pooled && g_full);
        Buf *wsb = new_buf("workspace", ws, true);
        if (epi_kind == CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL)
            st = convt3d_prepack_eval_weights(&g, reinterpret_cast<float *>(w->base), wp->base, nullptr);
        else
            st = convt3d_prepack_weights(&g, reinterpret_cast<float *>(w->base), wp->base, nullptr);
        if (st) fail("prepack status %d", st);
        st = convt3d_fused(reinterpret_cast<float *>(x->base), wp->base, reinterpret_cast<float *>(bias->base), &g, &e,
                           reinterpret_cast<float *>(out->base), wsb->base, ws, nullptr);
        if (st) fail("convt3d_fused status %d (%s)", st, convt3d_status_string(st));
        if (!pooled) check_coverage(out, oelems);
        int replayed = 1;

        // every plan convt3d_autotune may time: the candidates, and each one's
        // other border segmentations (its second stage)
        if (candidates && epi_kind != CONVT3D_EPI_SCALE_BN_EVAL_AVGPOOL) {
            std::vector<Plan> cands;
            if (plan_candidates(&g, &e, kTuneCandidates, &cands) != CONVT3D_OK) fail("plan_candidates failed");
            std::vector<Plan> all = cands;
            for (const Plan &c : cands) {
                std::vector<Plan> alt;
                if (plan_candidates(&g, &e, kTuneBorderAlternatives, &alt, &c) == CONVT3D_OK)
                    all.insert(all.end(), alt.begin(), alt.end());
            }
            g_full = false;  // the plan convt3d_fused runs was checked lane by lane above
            for (Plan &pl : all) {
                if (pl.ws_bytes > ws) fail("candidate needs %zu workspace bytes, more than the %zu reported", pl.ws_bytes, ws);
                pl.e = e;
                reset_tracking();
                ConvParams cp;
                fill_conv_params(pl, &cp);
                const bool stats_k = epi_kind == CONVT3D_EPI_RELU_GROUPNORM || epi_kind == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL;
                const int launches = pl.group_launch ? 1 : pl.G;
                for (int gi = 0; gi < launches; ++gi) {
                    cp.x = reinterpret_cast<float *>(x->base) + (size_t)gi * pl.cig * g.d * g.h * g.w;
                    cp.wp = reinterpret_cast<float *>(wp->base) + (size_t)gi * pl.packed_floats;
                    cp.bias = reinterpret_cast<float *>(bias->base) + (size_t)gi * pl.cog;
                    cp.out = pooled ? reinterpret_cast<float *>(out->base)
                                    : reinterpret_cast<float *>(out->base) + (size_t)gi * pl.cog * pl.S;
                    cp.partials = stats_k ? reinterpret_cast<float *>(wsb->base + pl.ws_partials) + (size_t)gi * pl.cog * pl.tiles_per_n * 2
                                          : nullptr;
                    replay_conv(pl, cp);
                }
                if (!pooled) check_coverage(out, oelems);
                if (epi_kind == CONVT3D_EPI_RELU_GROUPNORM)
                    launch_gn_finalize(reinterpret_cast<float *>(wsb->base + pl.ws_partials), g.n, (int)pl.tiles_per_n,
                                       g.cout, gn_groups, cp.gn_block8 ? 8 : 1, 1.0, 1e-5f, e.gamma, e.beta,
                                       reinterpret_cast<float *>(wsb->base + pl.ws_ab), e.stats_out, nullptr,
                                       reinterpret_cast<float *>(bias->base), 1.0, nullptr);
                if (epi_kind == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL)
                    launch_bn_finalize(reinterpret_cast<float *>(wsb->base + pl.ws_partials), g.n, (int)pl.tiles_per_n,
                                       g.cout, 1.0, e, reinterpret_cast<float *>(out->base), nullptr,
                                       reinterpret_cast<float *>(bias->base), nullptr);
                ++replayed;
                if (g_errors) break;
            }
        }
        if (g_errors) {
            std::printf("FAIL %s: %d errors; first: %s (plan variant %d split %d)\n", name, g_errors,
                        g_first_error.c_str(), info.variant, info.border_split);
            ++failed;
        } else {
            std::printf("ok %s: plan %d,%d,%d,%d,%d,%d,%d ploop %d, %d plans replayed, %lld checks\n", name, info.variant,
                        info.waves_co, info.tile_q[0], info.tile_q[1], info.tile_q[2], info.ci_chunk,
                        info.border_split, info.phase_loop, replayed, g_checks);
        }
        std::fflush(stdout);
        free_bufs();
    }
    std::printf("%d cases, %d failed\n", cases, failed);
    return failed ? 1 : 0;
}
