// HIP kernels of libconvt3d for gfx950 (CDNA4, wave64).
//
//  * prepack_kernel      -- nn.ConvTranspose3d weight [Cin, Cout, k, k, k] to
//                           per-stride-phase MFMA A-operand order.
//  * convt3d_mfma_kernel -- the transposed convolution as an output-stationary
//                           implicit GEMM per stride phase on FP32 MFMA
//                           (v_mfma_f32_32x32x2_f32), input halo staged in LDS,
//                           with the epilogue fused on the accumulators:
//                           bias (+ReLU) store with per-tile channel sums for
//                           GroupNorm, in-register channel softmax + sigmoid,
//                           or per-tile channel sums of scale*y for BatchNorm.
//
// The statistics, normalisation and standalone epilogue passes that run after
// this kernel are in epilogue.hip.
//
// MFMA 32x32x2 f32 operand layout (checked on the device): lane l supplies
// A[row = l%32][k = l/32] and B[k = l/32][col = l%32]; accumulator register r
// of lane l holds D[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].  Rows are
// output channels, columns are output voxels, k runs over (input channel, tap).
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "conv_index.hpp"
#include "convt3d_internal.hpp"

namespace convt3d {

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32x32x2(float a, float b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Cross-lane sums and maxima without the LDS crossbar: gfx950's lane-half
// swaps (v_permlane32_swap: lanes l and l ^ 32; v_permlane16_swap: rows of 16
// lanes, l and l ^ 16) and DPP row rotations.  The swap of v with itself
// leaves v's lower half in both halves of the first result and its upper half
// in both halves of the second, so their sum (or maximum) is v + v[l ^ 32] in
// every lane, the same bits as adding the partner's value.
__device__ __forceinline__ float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v + v of lane l - N within its row of 16 lanes (DPP row rotation)
template <int N>
__device__ __forceinline__ float add_row_ror(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
// Sum over the wave's 64 lanes.  Every lane ends with a sum of all 64 values,
// but the rotations add them in an order that depends on the lane: only one
// lane's result is to be used.
__device__ __forceinline__ float wave_sum(float v) {
    v = add_xor32(v);
    v = add_xor16(v);
    v = add_row_ror<8>(v);
    v = add_row_ror<4>(v);
    v = add_row_ror<2>(v);
    return add_row_ror<1>(v);
}

// ---------------------------------------------------------------------------
// Weight pre-pack of one channel group.  Packed order per phase:
// [co_block][octet][tap][lane][4] (as float4 groups [co_block][octet*ntaps +
// tap][lane]); element e of lane l of group (octet, tap) is
// w[ci = 8*octet + 2*e + l/32][co = 32*co_block + l%32] at kernel tap
// (r_d + ts_d*j_d, r_h + ts_h*j_h, r_w + ts_w*j_w), zero outside [0, Cin) x [0, Cout).
struct PackParams {
    const float *w;
    float *wp;
    int Cin, Cout, cb_total, nph;
    int k3[3], s3[3], ts[3];
    int pr[3][kMaxStride], pJ[3][kMaxStride];
    int ntaps[kMaxPhases], steps4[kMaxPhases], wp_off[kMaxPhases];
    int total4;
};

__global__ __launch_bounds__(256) void prepack_kernel(const PackParams P) {
    for (int i4 = blockIdx.x * blockDim.x + threadIdx.x; i4 < P.total4; i4 += gridDim.x * blockDim.x) {
        const int f = i4 * 4;
        int ph = 0;
        for (int q = 0; q < P.nph; ++q) {
            const int beg = P.wp_off[q];
            const int end = beg + P.cb_total * P.steps4[q] * 256;
            if (f >= beg && f < end) { ph = q; break; }
        }
        const int local = (f - P.wp_off[ph]) >> 2;
        const int lane = local & 63;
        const int t = local >> 6;
        const int steps4 = P.steps4[ph];
        const int G = t % steps4;
        const int cb = t / steps4;
        const int ntp = P.ntaps[ph];
        const int octet = G / ntp, tap = G % ntp;
        const int sh = P.s3[1], sw = P.s3[2];
        const int rd = ph / (sh * sw), rh = (ph / sw) % sh, rw = ph % sw;
        const int Jh = P.pJ[1][rh], Jw = P.pJ[2][rw];
        const int jw = tap % Jw, jh = (tap / Jw) % Jh, jd = tap / (Jw * Jh);
        const int kd = P.pr[0][rd] + P.ts[0] * jd, kh = P.pr[1][rh] + P.ts[1] * jh, kw = P.pr[2][rw] + P.ts[2] * jw;
        const int co = cb * 32 + (lane & 31);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ci = octet * 8 + 2 * e + (lane >> 5);
            v[e] = (ci < P.Cin && co < P.Cout)
                       ? P.w[((((size_t)ci * P.Cout + co) * P.k3[0] + kd) * P.k3[1] + kh) * P.k3[2] + kw]
                       : 0.0f;
        }
        *reinterpret_cast<float4 *>(P.wp + f) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// ---------------------------------------------------------------------------
// Transposed convolution on FP32 MFMA.
//
// Workgroup = 4 waves = WCO (co direction) x WPOS (position direction).  It
// owns: one sample n, one (rho_d, rho_h) phase pair (every pair with the
// phase-group loop), NPH consecutive w-phases, a box of TQd x TQh x TQw
// stride-phase positions q, and WCO*CBW blocks of 32 output channels.  Each
// wave owns CBW co-blocks x PBW blocks of 32 positions for each of its NPH
// w-phases.  Input channels are consumed in chunks of CI_T: the input halo of
// the box for those channels is staged in LDS, then every live tap of every
// phase runs 4 MFMA k-steps per 8 input channels.  With channel groups, grid z
// is sample * G + group and x, w, bias, out and partials are offset to the
// group's channels (Cout_total is the row stride); when that grid would be too
// tall the host launches once per group with offset pointers and G = 1.
// Minimum waves per SIMD, i.e. the register budget of each variant.  Four
// position blocks of one co block (64 accumulators, 16 B registers) may use up
// to 170 VGPRs (three waves) rather than being held to 128 (four), where an
// earlier form spilled in its chunk prologue; it now needs about 125 and runs
// four waves per SIMD.
template <int CBW, int NPH, int PBW, bool SM, bool PL, bool RP>
__global__ __launch_bounds__(kBlockThreads, RP ? 2 : (SM && CBW == 4) ? (NPH * PBW == 1 ? 2 : 1)
                                          : (CBW * NPH * PBW <= 2) ? 6
                                          : (CBW * NPH * PBW <= 4) ? 3
                                          : (CBW * NPH * PBW <= 8) ? 2 : 1)
void convt3d_mfma_kernel(const ConvParams P) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
    const int wco = wave % P.WCO;
    const int wpos = wave / P.WCO;

    // ---- workgroup -> work item (XCD-contiguous order), then its tile
    const ix::WorkItem wi =
        ix::work_item(P, blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gridDim.x, gridDim.y,
                      gridDim.z);
    const int bx = wi.bx, n = wi.n, grp = wi.grp, co_tile = wi.co_tile, wgrp = wi.wgrp;
    const ix::TileBox tb = ix::tile_box(P, bx);
    const int sd = P.s3[0], sh = P.s3[1], sw = P.s3[2];
    const int ed = P.pe[0], eh = P.pe[1], ew = P.pe[2];  // input step per tap index

    const int TQd = tb.TQd, TQh = tb.TQh, TQw = tb.TQw;
    const int q0d = tb.q0d, q0h = tb.q0h, q0w = tb.q0w;
    // extent of this tile inside its region (the box may overhang the region end)
    const int TQd_e = tb.TQd_e, TQh_e = tb.TQh_e, TQw_e = tb.TQw_e;

    // (rho_d, rho_h) phase groups of this workgroup: one (from the grid), or all
    // sd*sh of them over one staged halo when the whole channel range fits in
    // one LDS chunk.  The staged box is the union of the groups' footprints.
    constexpr bool ploop = PL;  // == (P.phase_loop != 0): the launcher picks the instantiation
    const int npg = ploop ? sd * sh : 1;
    const int pg0 = ploop ? 0 : wi.pg;
    int lo_d_rel, lo_h_rel, HD, HH;
    ix::halo_dh(P, pg0, npg, TQd, TQh, lo_d_rel, HD, lo_h_rel, HH);
    int Jw[NPH], cw[NPH], rw[NPH];
    int lo_w_rel = INT_MAX, hi_w_rel = INT_MIN;
#pragma unroll
    for (int p = 0; p < NPH; ++p) {
        rw[p] = wgrp * NPH + p;
        ix::w_phase(P, rw[p], TQw, Jw[p], cw[p], lo_w_rel, hi_w_rel);
    }
    const bool w_taps = ix::w_halo_close(TQw, lo_w_rel, hi_w_rel);

    // ---- halo box in input coordinates
    const int HW = hi_w_rel - lo_w_rel + 1;
    const int lo_d = q0d + lo_d_rel;
    const int lo_h = q0h + lo_h_rel;
    const int lo_w = q0w + lo_w_rel;
    int jw_lo[NPH], jw_hi[NPH];
#pragma unroll
    for (int p = 0; p < NPH; ++p) ix::tap_range(q0w, TQw_e, cw[p], ew, Jw[p], P.W, jw_lo[p], jw_hi[p]);

    // ---- LDS layout of a staged chunk: float4 [octet][k-row h][d][h][w].  The
    // lanes that feed MFMA k-row h (h = lane/32) need channels h, h+2, h+4, h+6
    // of an octet for the 4 k-steps of a group: they sit in one float4, read
    // with one 16-byte LDS read, and the 32 lanes of a k-row read consecutive
    // float4s along w (no bank conflicts).
    const int SLAB = HD * HH * HW;  // halo positions per octet
    const int slab2 = __builtin_amdgcn_readfirstlane(2 * SLAB);  // B offset per octet pair, scalar
    const int vol = TQd * TQh * TQw;
    const int plane = TQh * TQw;
    // The tile position of a lane's column in position block pb; decoded again
    // where it is needed (from an opaque copy of the lane's column index, so
    // the decode is not hoisted and kept live across the MFMA loop).
    auto decode_pos = [&](int pb, int &td, int &th, int &tw) -> bool {
        int c = col;
        asm volatile("" : "+v"(c));
        return ix::pos_decode(wpos * PBW + pb, c, vol, plane, TQw, TQd_e, TQh_e, TQw_e, td, th, tw);
    };
    int lane_off[PBW];  // float4 index of the lane's B reads at tap offset 0
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        int td, th, tw;
        decode_pos(pb, td, th, tw);
        lane_off[pb] = ix::b_lane_off(half, SLAB, td, th, tw, HH, HW);
    }

    const int CO_T = P.WCO * CBW;                   // co blocks per workgroup
    const int cb0 = co_tile * CO_T + wco * CBW;     // first co block of this wave
    const float4 *wp4 = reinterpret_cast<const float4 *>(P.wp + (size_t)grp * P.wpg);
    const int G4 = P.CI_T >> 3;
    const int DHWin = P.D * P.H * P.W;
    const float *xn = P.x + (size_t)n * P.x_nstride + (size_t)grp * P.xg;

    // ---- halo staging.  Thread t takes halo positions t, t + 256, ...; for each
    // it loads the 8 channels of every octet of the chunk and writes them as
    // two 16-byte LDS stores.  The loads are raw buffer loads: one descriptor
    // over the chunk's channel planes, formed once per chunk, with each
    // channel's plane offset in a scalar register and the position's byte
    // offset as the one vector operand.  (When the chunk's planes exceed what
    // 32-bit offsets reach, plain global loads with 64-bit addresses instead.)
    // A position outside the input gets an offset past the range and reads
    // zero; channels past Cin (a last, partial octet) are not
    // loaded and stage zero.  Every position of every chunk is written, so the
    // buffer needs no clearing.
    const int inc_w = kBlockThreads % HW, inc_h = (kBlockThreads / HW) % HH, inc_d = kBlockThreads / (HW * HH);
    const unsigned plane_bytes = 4u * (unsigned)DHWin;
    auto stage_t = [&](int chunk, auto per_plane) {
        constexpr bool kPlanes = decltype(per_plane)::value;
        int t = tid;  // opaque: the digits are formed here, not kept live across the MFMA loop
        asm volatile("" : "+v"(t));
        int w = t % HW, h = (t / HW) % HH, d = t / (HW * HH);
        const int oct0 = chunk * G4;
        // descriptors are formed from a base read into scalar registers (a
        // descriptor in vector registers needs a loop over its distinct values
        // at every load); the chunk's is formed here, outside the position loop
        auto scalar_ptr = [](uint64_t a) -> void * {
            // readfirstlane returns int: each half is taken as unsigned before
            // widening (a sign-extended low half would corrupt the high bits)
            return reinterpret_cast<void *>(ix::join_halves((unsigned)__builtin_amdgcn_readfirstlane((int)(a >> 32)),
                                                            (unsigned)__builtin_amdgcn_readfirstlane((int)a)));
        };
        const uint64_t xc = reinterpret_cast<uint64_t>(xn + (size_t)oct0 * 8 * DHWin);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            scalar_ptr(xc), (short)0, (int)ix::chunk_range_bytes(kPlanes ? 0 : P.CI_T, DHWin), 0x00020000);
        auto load = [&](int ch, unsigned vo) -> float {  // channel ch of the chunk at byte offset vo
            if constexpr (kPlanes) {
                return vo != ix::kHaloOutside ? reinterpret_cast<const float *>(xc)[(size_t)ch * DHWin + (vo >> 2)]
                                              : 0.0f;
            } else {
                return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, vo, ch * plane_bytes, 0));
            }
        };
        const int cin_left = __builtin_amdgcn_readfirstlane(P.Cin - oct0 * 8);
        for (int pos = t; pos < SLAB; pos += kBlockThreads) {
            const unsigned vo = ix::halo_src_off(lo_d + d, lo_h + h, lo_w + w, P.D, P.H, P.W);
            for (int g = 0; g < G4; ++g) {
                const int nch = cin_left - 8 * g;  // channels of the octet that exist (may be <= 0 past Cin)
                float v[8];
                if (nch >= 8) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) v[c] = load(8 * g + c, vo);
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) v[c] = c < nch ? load(8 * g + c, vo) : 0.0f;
                }
                float4 *l4 = reinterpret_cast<float4 *>(lds);
                l4[ix::stage_lds_index(g, SLAB, pos, 0)] = make_float4(v[0], v[2], v[4], v[6]);
                l4[ix::stage_lds_index(g, SLAB, pos, 1)] = make_float4(v[1], v[3], v[5], v[7]);
            }
            w += inc_w;
            if (w >= HW) { w -= HW; ++h; }
            h += inc_h;
            if (h >= HH) { h -= HH; ++d; }
            d += inc_d;
        }
    };
    auto stage = [&](int chunk) {
        if (P.plane_desc) stage_t(chunk, std::true_type{});
        else stage_t(chunk, std::false_type{});
    };
    stage(0);
    __syncthreads();

    // ---- register prefetch of the next channel chunk (RP kernels: one octet
    // per chunk, at most kRpPositions halo positions per thread, 32-bit plane
    // offsets; the planner keeps to these).  The loads of chunk k + 1 are
    // issued during chunk k's last MFMA groups, after those groups' A operands
    // are in registers, so nothing in the MFMA loop waits for them; after the
    // chunk's barrier they are written to LDS as staging would write them.
    // Every thread issues the same kRpPositions x 8 loads: positions past the
    // slab and channels past Cin take an offset past the range and load zero.
    static_assert(!RP || (CBW == 1 && NPH == 1 && PBW >= 4 && !SM && !PL), "prefetch builds: one form only");
    constexpr int RPN = RP ? kRpPositions : 1;
    float pf[RPN][8];
    // the thread's next halo position (digits w, h, d) and the chunk's
    // descriptor, set by prefetch_begin; prefetch_part issues the loads of the
    // thread's positions [i0, i1)
    int pw = 0, ph_ = 0, pd = 0, pnch = 0;
    uint64_t pxc = 0;
    auto prefetch_begin = [&](int chunk) {
        int t = tid;  // opaque, as in staging
        asm volatile("" : "+v"(t));
        pw = t % HW;
        ph_ = (t / HW) % HH;
        pd = t / (HW * HH);
        pxc = reinterpret_cast<uint64_t>(xn + (size_t)chunk * 8 * DHWin);
        pnch = __builtin_amdgcn_readfirstlane(P.Cin - chunk * 8);
    };
    auto prefetch_part = [&](auto i0c, auto i1c) {
        constexpr int i0 = decltype(i0c)::value, i1 = decltype(i1c)::value;
        const __amdgpu_buffer_rsrc_t pxr = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void *>(ix::join_halves((unsigned)__builtin_amdgcn_readfirstlane((int)(pxc >> 32)),
                                                     (unsigned)__builtin_amdgcn_readfirstlane((int)pxc))),
            (short)0, (int)ix::chunk_range_bytes(8, DHWin), 0x00020000);
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            const int pos = tid + i * kBlockThreads;
            const unsigned vo = pos < SLAB ? ix::halo_src_off(lo_d + pd, lo_h + ph_, lo_w + pw, P.D, P.H, P.W)
                                           : ix::kHaloOutside;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                pf[i][c] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(pxr, c < pnch ? vo : ix::kHaloOutside, c * plane_bytes, 0));
            pw += inc_w;
            if (pw >= HW) { pw -= HW; ++ph_; }
            ph_ += inc_h;
            if (ph_ >= HH) { ph_ -= HH; ++pd; }
            pd += inc_d;
        }
    };
    constexpr int RPH = RPN / 2;  // the loads go out in two bursts of at most 40 (the wait counter holds 63)
    auto prefetch = [&](int chunk) {
        prefetch_begin(chunk);
        prefetch_part(std::integral_constant<int, 0>{}, std::integral_constant<int, RPH>{});
        prefetch_part(std::integral_constant<int, RPH>{}, std::integral_constant<int, RPN>{});
    };
    auto write_prefetched = [&]() {
        float4 *l4 = reinterpret_cast<float4 *>(lds);
#pragma unroll
        for (int i = 0; i < RPN; ++i) {
            const int pos = tid + i * kBlockThreads;
            if (pos < SLAB) {
                l4[ix::stage_lds_index(0, SLAB, pos, 0)] = make_float4(pf[i][0], pf[i][2], pf[i][4], pf[i][6]);
                l4[ix::stage_lds_index(0, SLAB, pos, 1)] = make_float4(pf[i][1], pf[i][3], pf[i][5], pf[i][7]);
            }
        }
    };

    // a wave whose position blocks all lie past the box volume, or wholly in
    // the d-overhang at a region's end (d is the slowest index), runs no MFMAs
    const bool wave_live = min(vol, TQd_e * plane) > wpos * PBW * 32;

    // softmax kernels with up to two co blocks per wave start each accumulator
    // at its channel's bias (-inf for rows past Cout, whose packed weights are
    // zero): the softmax then needs no separate bias pass.  The same 16*CBW
    // values for every phase group, held in registers (with four co blocks
    // they would cost an occupancy step; those add the bias in the epilogue).
    constexpr bool BI = SM && CBW <= 2;
    float binit[BI ? CBW : 1][16];
    if constexpr (BI) {
#pragma unroll
        for (int c = 0; c < CBW; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = ix::acc_row(cb0 * 32, c, r) + 4 * half;
                binit[c][r] = row < P.Cout ? (P.bias ? P.bias[grp * P.Cout + row] : 0.0f) : -INFINITY;
            }
    }

  for (int pgi = 0; pgi < npg; ++pgi) {
    const int pg = pg0 + pgi;
    const int rho_h = pg % sh;
    const int rho_d = pg / sh;
    const int Jd = P.pJ[0][rho_d], cd = P.pc[0][rho_d];
    const int Jh = P.pJ[1][rho_h], ch = P.pc[1][rho_h];
    // ---- taps that touch the input for this box (border tiles skip the rest)
    int jd_lo, jd_hi, jh_lo, jh_hi;
    ix::tap_range(q0d, TQd_e, cd, ed, Jd, P.D, jd_lo, jd_hi);
    ix::tap_range(q0h, TQh_e, ch, eh, Jh, P.H, jh_lo, jh_hi);

    v16f acc[NPH][CBW][PBW];
#pragma unroll
    for (int p = 0; p < NPH; ++p)
#pragma unroll
        for (int c = 0; c < CBW; ++c)
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[p][c][pb][r] = BI ? binit[BI ? c : 0][r] : 0.0f;

    bool work = Jd > 0 && Jh > 0 && w_taps && jd_lo <= jd_hi && jh_lo <= jh_hi;
    {
        bool anyw = false;
#pragma unroll
        for (int p = 0; p < NPH; ++p) anyw = anyw || (Jw[p] > 0 && jw_lo[p] <= jw_hi[p]);
        work = work && anyw;
    }
    if (work) {
        for (int chunk = 0; chunk < P.nchunks; ++chunk) {
            if constexpr (!PL) {
                if (chunk > 0) {  // stage the next chunk while the workgroup waits
                    __syncthreads();
                    if constexpr (RP) write_prefetched();
                    else stage(chunk);
                    __syncthreads();
                }
            }
            // softmax kernels: waves in their MFMA loop issue before waves in the
            // (vector-ALU heavy) epilogue (measured +2 %; the other epilogues
            // lose 1-2 % because their staging waves then wait longer)
            if constexpr (SM) __builtin_amdgcn_s_setprio(1);
            bool pf_done = false;  // RP: this wave has issued the next chunk's prefetch
#pragma unroll
            for (int p = 0; p < NPH; ++p) {
                if (!wave_live || Jw[p] == 0 || jw_lo[p] > jw_hi[p]) continue;
                const int ph = (rho_d * sh + rho_h) * sw + rw[p];
                const int ntp = P.ntaps[ph];
                const int jwl = jw_lo[p], jwh = jw_hi[p], jwn = Jw[p], cwp = cw[p];
                // A operands of a group: 16 bytes per lane at (co block base +
                // group) of the packed weights, read as a raw buffer (stride 0,
                // no range limit, 32-bit data format) with the group offset in a
                // scalar register and the lane offset in a fixed vector register:
                // no vector address arithmetic per group
                __amdgpu_buffer_rsrc_t wr[CBW];
#pragma unroll
                for (int c = 0; c < CBW; ++c) {
                    const int cb = min(cb0 + c, P.cb_total - 1);
                    const float4 *base = wp4 + ix::a_block_base(P, ph, cb);
                    wr[c] = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, 0x7FFFFFF0, 0x00020000);
                }
                const int lane16 = lane * 16;
                typedef unsigned int u4v __attribute__((ext_vector_type(4)));
                auto aload = [&](int c, int gi) -> float4 {
                    const u4v v = __builtin_amdgcn_raw_buffer_load_b128(wr[c], lane16, gi * 16, 0);
                    return *reinterpret_cast<const float4 *>(&v);
                };
                const int n_it = (jd_hi - jd_lo + 1) * (jh_hi - jh_lo + 1) * (jwh - jwl + 1) * G4;
                // Iteration state (jd, jh, jw, g4) of the next group to load; every
                // group is 4 MFMA k-steps = 8 input channels of one tap.  gi: float4
                // index of its A operands; bo: float4 offset of its B operands.
                int jd = jd_lo, jh = jh_lo, jw = jwl, g4 = 0;
                auto next_group = [&](int &gi, int &bo) {
                    gi = ix::a_group_index(chunk, G4, g4, ntp, jd, Jh, jh, jwn, jw);
                    bo = ix::b_group_off(cd, ed, jd, lo_d_rel, ch, eh, jh, lo_h_rel, cwp, ew, jw, lo_w_rel, HH, HW,
                                         g4, slab2);
                    if (++g4 == G4) {
                        g4 = 0;
                        if (++jw > jwh) { jw = jwl; if (++jh > jh_hi) { jh = jh_lo; ++jd; } }
                    }
                };
                // One group = 4 MFMA k-steps; its B operands (4 per position block)
                // come from one 16-byte LDS read per position block, issued one
                // group ahead.
                const float4 *lds4 = reinterpret_cast<const float4 *>(lds);
                float4 aA[CBW], aB[CBW];
                int giA, boA, giB, boB;
                next_group(giA, boA);
#pragma unroll
                for (int c = 0; c < CBW; ++c) aA[c] = aload(c, giA);
                if constexpr (PBW >= 4) {
                    // One B register set: a position block's registers are refilled
                    // with the next group's B right after their last MFMA (k-step 3);
                    // the other position blocks' MFMAs cover the LDS latency.
                    float4 bq[PBW];
#pragma unroll
                    for (int pb = 0; pb < PBW; ++pb) bq[pb] = lds4[lane_off[pb] + boA];
                    auto group_mfma = [&](const float4 (&a)[CBW], int bo_next) {
#pragma unroll
                        for (int e = 0; e < 3; ++e)
#pragma unroll
                            for (int c = 0; c < CBW; ++c)
#pragma unroll
                                for (int pb = 0; pb < PBW; ++pb)
                                    acc[p][c][pb] = mfma32x32x2(a[c][e], bq[pb][e], acc[p][c][pb]);
#pragma unroll
                        for (int pb = 0; pb < PBW; ++pb) {
#pragma unroll
                            for (int c = 0; c < CBW; ++c)
                                acc[p][c][pb] = mfma32x32x2(a[c][3], bq[pb][3], acc[p][c][pb]);
                            bq[pb] = lds4[lane_off[pb] + bo_next];
                        }
                        __builtin_amdgcn_sched_group_barrier(0x008, 3 * CBW * PBW, 0);
#pragma unroll
                        for (int pb = 0; pb < PBW; ++pb) {
                            __builtin_amdgcn_sched_group_barrier(0x008, CBW, 0);  // CBW MFMAs
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
                        }
                    };
                    // RP kernels before a further chunk: the loop stops at an even
                    // group count n_main, leaving the last groups (up to kTail + 1)
                    // to a tail that prefetches the next chunk
                    constexpr int kTail = 4;
                    const bool tail_pf = RP && chunk + 1 < P.nchunks;
                    const int n_main = tail_pf ? (n_it > kTail ? ((n_it - kTail) & ~1) : 0) : n_it;
                    for (int it = 0; it < n_main; it += 2) {
                        if (it + 1 < n_it) next_group(giB, boB); else { giB = giA; boB = boA; }
#pragma unroll
                        for (int c = 0; c < CBW; ++c) aB[c] = aload(c, giB);
                        __builtin_amdgcn_sched_barrier(0);
                        group_mfma(aA, boB);
                        __builtin_amdgcn_sched_barrier(0);
                        if (it + 1 >= n_it) break;
                        if (it + 2 < n_it) next_group(giA, boA); else { giA = giB; boA = boB; }
#pragma unroll
                        for (int c = 0; c < CBW; ++c) aA[c] = aload(c, giA);
                        __builtin_amdgcn_sched_barrier(0);
                        group_mfma(aB, boA);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if constexpr (RP) {
                        if (tail_pf) {
                            // aA and bq hold group n_main; load the A operands of the
                            // (up to kTail) groups after it and wait for them, then
                            // issue the prefetch in two bursts between the tail's
                            // groups: no MFMA of the tail waits on a vector load
                            const int nt = n_it - n_main;  // 1 .. kTail + 1
                            float4 at[kTail][CBW];
                            int bo[kTail + 1];
                            bo[0] = boA;
#pragma unroll
                            for (int j = 1; j <= kTail; ++j) {
                                bo[j] = bo[j - 1];
                                if (j < nt) {
                                    int gi;
                                    next_group(gi, bo[j]);
#pragma unroll
                                    for (int c = 0; c < CBW; ++c) at[j - 1][c] = aload(c, gi);
                                }
                            }
                            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tail's A operands
                            __builtin_amdgcn_sched_barrier(0);
                            prefetch_begin(chunk + 1);
                            prefetch_part(std::integral_constant<int, 0>{}, std::integral_constant<int, RPH>{});
                            pf_done = true;
                            __builtin_amdgcn_sched_barrier(0);
                            group_mfma(aA, nt > 1 ? bo[1] : bo[0]);
                            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                            for (int j = 1; j <= kTail; ++j) {
                                if (j == kTail / 2) {
                                    prefetch_part(std::integral_constant<int, RPH>{}, std::integral_constant<int, RPN>{});
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                                if (j < nt) group_mfma(at[j - 1], j + 1 < nt ? bo[j + 1] : bo[j]);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                    }
                } else {
                    // Two B register sets: the next group's B is read before this
                    // group's MFMAs.
                    float4 bA[PBW], bB[PBW];
                    auto read_b = [&](float4 (&b)[PBW], int bo) {
#pragma unroll
                        for (int pb = 0; pb < PBW; ++pb) b[pb] = lds4[lane_off[pb] + bo];
                    };
                    auto group_mfma = [&](const float4 (&a)[CBW], const float4 (&b)[PBW]) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
#pragma unroll
                            for (int c = 0; c < CBW; ++c)
#pragma unroll
                                for (int pb = 0; pb < PBW; ++pb)
                                    acc[p][c][pb] = mfma32x32x2(a[c][e], b[pb][e], acc[p][c][pb]);
                    };
                    read_b(bA, boA);
                    for (int it = 0; it < n_it; it += 2) {
                        if (it + 1 < n_it) next_group(giB, boB); else { giB = giA; boB = boA; }
#pragma unroll
                        for (int c = 0; c < CBW; ++c) aB[c] = aload(c, giB);
                        read_b(bB, boB);
                        __builtin_amdgcn_sched_barrier(0);
                        group_mfma(aA, bA);
                        __builtin_amdgcn_sched_barrier(0);
                        if (it + 1 >= n_it) break;
                        if (it + 2 < n_it) next_group(giA, boA); else { giA = giB; boA = boB; }
#pragma unroll
                        for (int c = 0; c < CBW; ++c) aA[c] = aload(c, giA);
                        read_b(bA, boA);
                        __builtin_amdgcn_sched_barrier(0);
                        group_mfma(aB, bB);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            if constexpr (RP) {
                // waves that ran no MFMAs still stage their share of the next chunk
                if (chunk + 1 < P.nchunks && !pf_done) prefetch(chunk + 1);
            }
            if constexpr (SM) __builtin_amdgcn_s_setprio(0);
        }
    }

    // ------------------------------------------------------------------ epilogue
    // Accumulator register r of co block c holds output channel
    // row0 + 32c + 8(r/4) + r%4 + 4*half at the lane's column position.  Store
    // addresses are a wave-uniform row base (scalar registers) plus the lane's
    // byte offset, formed once per position block: no vector address math per
    // store.
    const int Do = P.Do, Ho = P.Ho, Wo = P.Wo;
    const int S = Do * Ho * Wo;  // the planner keeps 20*S (the largest byte offset) below 2^32
    unsigned vofs[NPH][PBW];     // byte offset of the lane's output from its row base
    bool ok[NPH][PBW];
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        int td, th, tw;
        const bool pos_ok = decode_pos(pb, td, th, tw);
        const int od = sd * (q0d + td) + rho_d;
        const int oh = sh * (q0h + th) + rho_h;
#pragma unroll
        for (int p = 0; p < NPH; ++p) {
            const int ow = sw * (q0w + tw) + rw[p];
            ok[p][pb] = pos_ok && od < Do && oh < Ho && ow < Wo;
            vofs[p][pb] = (unsigned)ix::out_voxel_off(half, S, od, Ho, oh, Wo, ow) * 4u;
        }
    }
    // both w-phases of a lane land in one aligned float pair (w even, w + 1)
    bool pair_ok[PBW];
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        pair_ok[pb] = false;
        if constexpr (NPH == 2)
            pair_ok[pb] = ok[0][pb] && ok[1][pb] && (Wo % 2 == 0);  // rw[0] is even when NPH == 2
    }
    const int Cout = P.Cout;
    // first output channel of the wave; inside the phase-group loop it is made
    // opaque so the row bases are formed here, not hoisted out of the loop and
    // kept live across the MFMAs
    int row0 = cb0 * 32;
    if constexpr (PL) asm volatile("" : "+s"(row0));
    const bool rows_full = row0 + CBW * 32 <= Cout;  // every accumulator row is a channel
    char *outb = reinterpret_cast<char *>(P.out + ((size_t)n * P.Cout_total + (size_t)grp * Cout) * S);
    auto row_u = [&](int c, int r) { return ix::acc_row(row0, c, r); };
    auto row_ok = [&](int c, int r) { return rows_full || row_u(c, r) + 4 * half < Cout; };
    auto rowp = [&](int c, int r) { return outb + (size_t)row_u(c, r) * S * 4; };
    // the bias of the lane's rows 4q .. 4q+3 of co block c (0 without bias and
    // for rows past Cout): the four loads are issued together and waited for
    // once.  The group offset is made opaque here so the loads stay in the
    // epilogue, not hoisted above the MFMA loop.
    auto bias_rows4 = [&](int c, int q, float (&bv)[4]) {
        if (P.bias) {
            int gofs = grp * Cout;
            asm volatile("" : "+s"(gofs));
            const float *b = P.bias + gofs;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row_u(c, 4 * q + i) + 4 * half;
                bv[i] = rows_full || row < Cout ? b[row] : 0.0f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = 0.0f;
        }
    };
    // the stores of one accumulator row (c, r) of position block pb.  The
    // softmax kernels write the final output, which nothing here reads again:
    // non-temporal stores (2 % faster on the 64-channel stride-2 layer); the
    // other kernels' y is read back by the normalise pass and stays cached.
    auto store_row = [&](char *rp, int pb, const float (&v)[NPH]) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        if constexpr (NPH == 2) {
            if (pair_ok[pb]) {
                f2 *dst = reinterpret_cast<f2 *>(rp + vofs[0][pb]);
                const f2 val = {v[0], v[1]};
                if constexpr (SM) __builtin_nontemporal_store(val, dst);
                else *dst = val;
                return;
            }
        }
#pragma unroll
        for (int p = 0; p < NPH; ++p)
            if (ok[p][pb]) {
                float *dst = reinterpret_cast<float *>(rp + vofs[p][pb]);
                if constexpr (SM) __builtin_nontemporal_store(v[p], dst);
                else *dst = v[p];
            }
    };

    if constexpr (SM) {
        // Channel softmax + sigmoid.  The wave holds every channel of its columns
        // (planner: WCO == 1 and CBW*32 >= Cout); lane l and lane l^32 hold
        // complementary halves.  Bias first (padding rows -> -inf, so they add
        // 0), unless the accumulators started at it.
        if constexpr (!BI) {
            // one row at a time: loading them in groups costs these kernels
            // (four co blocks, tight on registers) an occupancy step
#pragma unroll
            for (int c = 0; c < CBW; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float bo = P.bias ? P.bias[grp * Cout + row_u(c, r) + 4 * half] : 0.0f;
                    const float bco = row_ok(c, r) ? bo : -INFINITY;
#pragma unroll
                    for (int p = 0; p < NPH; ++p)
#pragma unroll
                        for (int pb = 0; pb < PBW; ++pb) acc[p][c][pb][r] += bco;
                }
        }
        // exp(x) = 2^(x*log2 e) on the hardware exp2, 1/x on the hardware
        // reciprocal (about 1 ulp each); the max is taken on the scaled values.
        constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
        for (int p = 0; p < NPH; ++p)
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                float m = -INFINITY;
#pragma unroll
                for (int c = 0; c < CBW; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[p][c][pb][r]);
                m = max_xor32(m);
                const float ml = m * kLog2e;
                float sum = 0.0f;
#pragma unroll
                for (int c = 0; c < CBW; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        // 0 for padding rows (-inf)
                        const float e = __builtin_amdgcn_exp2f(fmaf(acc[p][c][pb][r], kLog2e, -ml));
                        acc[p][c][pb][r] = e;
                        sum += e;
                    }
                sum = add_xor32(sum);
                // sigmoid(q) for the probability q = e/sum in [0, 1]: 1/2 + q R(q^2)
                // with the odd polynomial of kSigmoidOdd (|error| < 1.2e-7; the
                // coefficients are printed by sigmoid_poly.py beside this file),
                // as 1/2 + e R'(e^2) with R' = sum_k (r_k / sum^(2k+1)) (e^2)^k.
                const float inv = __builtin_amdgcn_rcpf(sum);
                const float inv2 = inv * inv;
                float d[4];
                float ik = inv;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    d[k] = kSigmoidOdd[k] * ik;
                    ik *= inv2;
                }
#pragma unroll
                for (int c = 0; c < CBW; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = acc[p][c][pb][r];
                        const float e2 = e * e;
                        float t = d[3];
#pragma unroll
                        for (int k = 2; k >= 0; --k) t = fmaf(t, e2, d[k]);
                        acc[p][c][pb][r] = fmaf(t, e, 0.5f);
                    }
            }
        // stores: bounds-checked non-temporal buffer stores, one descriptor per
        // accumulator row covering the bytes of its existing channels.  A lane
        // whose output does not exist gets an offset past that range and the
        // hardware drops its store: no per-lane branches.  With two w-phases a
        // lane holds outputs at w and w+1, stored as one float pair; lanes
        // where only one of them exists store singly, in a second sequence a
        // wave runs only when it has such a lane.
        typedef unsigned int u2v __attribute__((ext_vector_type(2)));
        unsigned so[NPH][PBW], po[PBW];
        bool singles = false;
#pragma unroll
        for (int pb = 0; pb < PBW; ++pb) {
            po[pb] = ix::kDropOffset;
            if constexpr (NPH == 2) po[pb] = pair_ok[pb] ? vofs[0][pb] : ix::kDropOffset;
#pragma unroll
            for (int p = 0; p < NPH; ++p) {
                const bool single = ok[p][pb] && (NPH == 1 || !pair_ok[pb]);
                so[p][pb] = single ? vofs[p][pb] : ix::kDropOffset;
                singles = singles || (NPH == 2 && single);
            }
        }
        const bool any_single = NPH == 1 || __any(singles);
#pragma unroll
        for (int c = 0; c < CBW; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    rowp(c, r), (short)0, (int)ix::row_pair_bytes(row_u(c, r), Cout, S), 0x00020000);
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb) {
                    if constexpr (NPH == 2) {
                        const float2 pv = make_float2(acc[0][c][pb][r], acc[1][c][pb][r]);
                        __builtin_amdgcn_raw_buffer_store_b64(*reinterpret_cast<const u2v *>(&pv), rs, po[pb], 0, 2);
                    }
                    if (any_single)
#pragma unroll
                        for (int p = 0; p < NPH; ++p)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[p][c][pb][r]), rs, so[p][pb], 0,
                                                                  2);
                }
            }
    } else {
        // bias (+ReLU) and store, or scale; per-channel sums over the tile: the
        // lane's columns, then the 32 columns of each half (xor-shuffle
        // butterfly, or per 8-channel block for GroupNorm: lane-half swaps and
        // row rotations over the whole wave), then the waves
        // (LDS), one (sum, sum of squares) per (tile, channel).  The sums are
        // of v - pivot with a per-channel pivot near the channel's values, so
        // a large common offset does not cancel in the fp32 sum of squares:
        // GroupNorm relu(bias) (of the block's first channel for block sums),
        // BatchNorm scale*bias (the sums are then of scale*acc); the statistics
        // merge adds the pivots back in fp64.
        const bool gn = P.epi == CONVT3D_EPI_RELU_GROUPNORM;
        const bool bn = P.epi == CONVT3D_EPI_SCALE_BN_TRAIN_AVGPOOL;
        const float scale = P.scale;
        const int CO32 = CO_T * 32;
        float *red = lds + P.red_off;  // [WPOS][CO_T*32][2], after the halo
        if (gn || bn) __syncthreads();  // the previous phase group's readers are done
        const bool blk8 = gn && P.gn_block8;
        if (blk8) {
            // GroupNorm over groups of whole 8-channel blocks: a lane's four rows
            // of block q (channels 8q + r%4 + 4*half) are summed first, then the
            // block sum over all 64 lanes; one (sum, sum of squares) per
            // (tile, block), kept at the block's first channel (the other seven
            // channels' partials are not written)
#pragma unroll
            for (int c = 0; c < CBW; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float bv[4];
                    bias_rows4(c, q, bv);
                    const bool bok = row_ok(c, 4 * q);  // whole block in range (Cout % 8 == 0)
                    // the block's pivot: relu(bias) of its first channel (wave-uniform)
                    const float pvt = bok && P.bias ? fmaxf(P.bias[grp * Cout + row0 + c * 32 + 8 * q], 0.0f) : 0.0f;
                    float b1 = 0.0f, b2 = 0.0f;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = 4 * q + rr;
                        const float bco = bok ? bv[rr] : 0.0f;
                        char *rp = rowp(c, r);
#pragma unroll
                        for (int pb = 0; pb < PBW; ++pb) {
                            float v[NPH];
#pragma unroll
                            for (int p = 0; p < NPH; ++p) {
                                v[p] = fmaxf(acc[p][c][pb][r] + bco, 0.0f);
                                const float vm = ok[p][pb] ? v[p] - pvt : 0.0f;
                                b1 += vm;
                                b2 = fmaf(vm, vm, b2);
                            }
                            if (bok) store_row(rp, pb, v);
                        }
                    }
                    b1 = wave_sum(b1);  // lane 0's sums are the block's
                    b2 = wave_sum(b2);
                    if (lane == 0 && bok) {
                        const int row = (wco * CBW + c) * 32 + 8 * q;
                        red[(wpos * CO32 + row) * 2 + 0] = b1;
                        red[(wpos * CO32 + row) * 2 + 1] = b2;
                    }
                }
        } else
#pragma unroll
        for (int c = 0; c < CBW; ++c) {
            // per-row sums x[r] (sum) and x[16 + r] (sum of squares) of the lane
            float x[32];
            float bv[4];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // BatchNorm sums z - scale*bias = scale*acc: its bias stays out
                if (r % 4 == 0) {
                    if (bn) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) bv[i] = 0.0f;
                    } else {
                        bias_rows4(c, r / 4, bv);
                    }
                }
                const bool cok = row_ok(c, r);
                // GroupNorm sums relu(acc + bias) - relu(bias)
                const float bco = cok ? bv[r % 4] : 0.0f;
                float a1 = 0.0f, a2 = 0.0f;
                char *rp = rowp(c, r);
#pragma unroll
                for (int pb = 0; pb < PBW; ++pb) {
                    float v[NPH];
#pragma unroll
                    for (int p = 0; p < NPH; ++p) {
                        v[p] = acc[p][c][pb][r] + bco;
                        if (gn) v[p] = fmaxf(v[p], 0.0f);
                        const float d = fmaf(v[p], bn ? scale : 1.0f, gn ? -fmaxf(bco, 0.0f) : 0.0f);
                        const float vm = ok[p][pb] ? d : 0.0f;
                        a1 += vm;
                        a2 = fmaf(vm, vm, a2);
                    }
                    if (cok && !bn) store_row(rp, pb, v);
                }
                x[r] = a1;
                x[16 + r] = a2;
            }
            if (gn || bn) {
                // butterfly reduce-scatter over the 32 lanes of a half: at each
                // step a lane keeps one half of its values, sends the other half
                // to lane ^ m and adds what it receives; afterwards lane col holds
                // the half's total of value col (row col % 16, sum or square sum)
#pragma unroll
                for (int m = 16, k = 16; m >= 1; m >>= 1, k >>= 1) {
                    const bool up = (col & m) != 0;
#pragma unroll
                    for (int j = 0; j < k; ++j) {
                        const float keep = up ? x[j + k] : x[j];
                        const float send = up ? x[j] : x[j + k];
                        x[j] = keep + __shfl_xor(send, m);
                    }
                }
                const int r = col & 15;
                const int row = (wco * CBW + c) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (row_ok(c, r)) red[(wpos * CO32 + row) * 2 + (col >> 4)] = x[0];
            }
        }
        if (gn || bn) {
            __syncthreads();
            const int tile = ix::partial_tile(P, rho_d, rho_h, wgrp, bx);
            for (int row = tid; row < CO32; row += blockDim.x) {
                const int co = co_tile * CO32 + row;
                if (co >= Cout) continue;
                // block sums sit at each block's first channel, and the merge
                // reads only those
                if (blk8 && (row & 7) != 0) continue;
                float t1 = 0.0f, t2 = 0.0f;
                for (int w = 0; w < P.WPOS; ++w) {
                    t1 += red[(w * CO32 + row) * 2 + 0];
                    t2 += red[(w * CO32 + row) * 2 + 1];
                }
                float *pp = P.partials + ix::partial_offset(n, P.Cout_total, grp * Cout + co, P.tiles_per_n, tile);
                pp[0] = t1;
                pp[1] = t2;
            }
        }
    }
  }  // phase groups
}

// ---------------------------------------------------------------------------
// launchers

static int grid_for(int64_t items, int per_block, int cap) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

int launch_prepack(const Plan &pl, const float *w, float *wp, void *stream) {
    PackParams P{};
    P.w = w;
    P.wp = wp;
    P.Cin = pl.cig;
    P.Cout = pl.cog;
    for (int d = 0; d < 3; ++d) {
        P.k3[d] = pl.g.k[d];
        P.s3[d] = pl.s3[d];
        P.ts[d] = pl.ts[d];
    }
    P.cb_total = pl.cb_total;
    P.nph = pl.nph;
    for (int d = 0; d < 3; ++d)
        for (int r = 0; r < kMaxStride; ++r) {
            P.pr[d][r] = pl.ph[d][r].r;
            P.pJ[d][r] = pl.ph[d][r].J;
        }
    for (int q = 0; q < kMaxPhases; ++q) {
        P.ntaps[q] = pl.ntaps[q];
        P.steps4[q] = pl.steps4[q];
        P.wp_off[q] = (int)pl.wp_off[q];
    }
    P.total4 = (int)(pl.packed_floats / 4);
    if (P.total4 == 0) return (int)hipSuccess;
    hipLaunchKernelGGL(prepack_kernel, dim3(grid_for(P.total4, 256, 65536)), dim3(256), 0,
                       (hipStream_t)stream, P);
    return (int)hipGetLastError();
}

template <int CBW, int NPH, int PBW, bool SM, bool PL, bool RP = false>
static int launch_conv_t(const Plan &pl, const ConvParams &cp, void *stream) {
    auto fn = convt3d_mfma_kernel<CBW, NPH, PBW, SM, PL, RP>;
    // the dynamic-LDS limit is a per-device attribute of the function: set it
    // once on every device the kernel runs on (bit d: done on device d)
    static std::atomic<uint64_t> attr_done{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return (int)err;
    const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
    if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  kMaxLdsBytes);
        if (err != hipSuccess) return (int)err;
        attr_done.fetch_or(bit, std::memory_order_acq_rel);
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)pl.grid_x, (unsigned)pl.grid_y, (unsigned)pl.grid_z),
                       dim3(kBlockThreads), pl.lds_bytes, (hipStream_t)stream, cp);
    return (int)hipGetLastError();
}

int launch_conv(const Plan &pl, const ConvParams &cp, void *stream) {
    const Variant v = kVariants[pl.variant];
    const bool pl_ = pl.phase_loop != 0;
    // the register-prefetch build (its own variant entry)
    if (v.prefetch) {
        if (v.CBW == 1 && v.NPH == 1 && v.PBW == 4 && !v.softmax && !pl_)
            return launch_conv_t<1, 1, 4, false, false, true>(pl, cp, stream);
        return (int)hipErrorInvalidValue;
    }
#define CONVT3D_VARIANT(a, b, c, d) \
    if (v.CBW == a && v.NPH == b && v.PBW == c && v.softmax == d && !pl_) \
        return launch_conv_t<a, b, c, d, false>(pl, cp, stream);
#define CONVT3D_VARIANT_PL(a, b, c, d) \
    if (v.CBW == a && v.NPH == b && v.PBW == c && v.softmax == d && pl_) \
        return launch_conv_t<a, b, c, d, true>(pl, cp, stream);
    CONVT3D_VARIANT(1, 1, 8, false)
    CONVT3D_VARIANT(1, 1, 4, false)
    CONVT3D_VARIANT(1, 1, 2, false)
    CONVT3D_VARIANT(1, 2, 4, false)
    CONVT3D_VARIANT(1, 2, 2, false)
    CONVT3D_VARIANT(1, 1, 4, true)
    CONVT3D_VARIANT(1, 1, 2, true)
    CONVT3D_VARIANT(1, 2, 2, true)
    CONVT3D_VARIANT(2, 1, 4, true)
    CONVT3D_VARIANT(2, 2, 2, true)
    CONVT3D_VARIANT(2, 1, 2, true)
    CONVT3D_VARIANT(2, 2, 1, true)
    CONVT3D_VARIANT(4, 1, 2, true)
    CONVT3D_VARIANT(4, 2, 1, true)
    CONVT3D_VARIANT(4, 1, 1, true)
    // phase-group loop instantiations (stride > 1, one channel chunk)
    CONVT3D_VARIANT_PL(1, 1, 4, false)
    CONVT3D_VARIANT_PL(1, 2, 2, false)
    CONVT3D_VARIANT_PL(1, 2, 4, false)
    CONVT3D_VARIANT_PL(1, 1, 2, true)
    CONVT3D_VARIANT_PL(1, 2, 2, true)
    CONVT3D_VARIANT_PL(2, 2, 2, true)
    CONVT3D_VARIANT_PL(2, 2, 1, true)
    CONVT3D_VARIANT_PL(2, 1, 2, true)
    CONVT3D_VARIANT_PL(4, 2, 1, true)
    CONVT3D_VARIANT_PL(4, 1, 1, true)
#undef CONVT3D_VARIANT
#undef CONVT3D_VARIANT_PL
    return (int)hipErrorInvalidValue;
}

}  // namespace convt3d
