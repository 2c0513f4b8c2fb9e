// kernels_fp.h -- the fp16/bf16 GEMM kernels (direct rungs for decode-
// adjacent M and skinny N, streaming tiles for mid and long prefill, the K
// split across workgroups, grouped per-expert tiles) and the template that
// launches a Plan's rung.  Included by the instantiation units only.
#pragma once

#include "common.h"
#include "plan.h"

namespace qg {

// ---------------------------------------------------------------------------
// Direct kernel: decode-adjacent M and skinny N.
//
// Each wave unpacks its weight fragments straight into VGPRs and reuses them
// for RB row blocks of 16 tokens; the a.kw waves of a workgroup split the K
// loop (the K-parallel shape of the batched-prefill post: many lanes share a
// row reduction, then one reduction per output at the end) and combine their
// partial sums through LDS.  The raw weight bytes and activation fragments of
// chunk c+1 are in flight while chunk c is unpacked and multiplied.  Grid:
// x = panel groups of PN panels, y = row groups of 16*RB rows.
// ---------------------------------------------------------------------------
// One workgroup: rows m0 .. m0+16*RB-1 (those below a.M) of panels p0 ..
// p0+PN-1; a.kw waves split K and reduce through LDS.
template <int FMT, int DT, int RB, int PN, int XL>
__device__ __forceinline__ void direct_body(const Args &a, int p0, int m0)
{
    using XA = XLay<XL>;
    extern __shared__ f32x4 red[];  // [kw][PN*RB][64]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int nch = a.K / kChunk;
    const int cb = (int)((long long)nch * w / a.kw), ce = (int)((long long)nch * (w + 1) / a.kw);

    f32x4 acc[PN][RB];
#pragma unroll
    for (int pn = 0; pn < PN; pn++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++) acc[pn][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t *xrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        int r = m0 + 16 * rb + col;
        r = r < a.M ? r : a.M - 1;  // clamped rows are computed and discarded
        xrow[rb] = XA::row(a, r) + XA::off(32 * g);
    }
    RunSrc<FMT> src[PN];
#pragma unroll
    for (int pn = 0; pn < PN; pn++) {
        const int p = p0 + pn;
        src[pn].init(a, p < a.np ? p : a.np - 1, g, col);
    }

    RunRaw<FMT> raw[PN];
    u32x4 xf[RB][4];
    if (cb < ce) {
#pragma unroll
        for (int pn = 0; pn < PN; pn++) src[pn].load(cb, raw[pn]);
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int i = 0; i < 4; i++) xf[rb][i] = *(const u32x4 *)(xrow[rb] + XA::chunk(cb) + XA::off(8 * i));
    }
    for (int c = cb; c < ce; c++) {
        u32x4 wf[PN][4];
#pragma unroll
        for (int pn = 0; pn < PN; pn++) unpack_run<FMT, DT>(raw[pn], src[pn], c, wf[pn]);
        u32x4 xc[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int i = 0; i < 4; i++) xc[rb][i] = xf[rb][i];
        if (c + 1 < ce) {  // prefetch chunk c+1 while this one is multiplied
#pragma unroll
            for (int pn = 0; pn < PN; pn++) src[pn].load(c + 1, raw[pn]);
#pragma unroll
            for (int rb = 0; rb < RB; rb++)
#pragma unroll
                for (int i = 0; i < 4; i++) xf[rb][i] = *(const u32x4 *)(xrow[rb] + XA::chunk(c + 1) + XA::off(8 * i));
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int pn = 0; pn < PN; pn++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[pn][rb] = mma<DT>(wf[pn][i], xc[rb][i], acc[pn][rb]);
    }

    if (a.kw == 1) {
#pragma unroll
        for (int pn = 0; pn < PN; pn++)
#pragma unroll
            for (int rb = 0; rb < RB; rb++) store_block<DT>(a, acc[pn][rb], m0 + 16 * rb, 16 * (p0 + pn), lane);
        return;
    }
#pragma unroll
    for (int pn = 0; pn < PN; pn++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++) red[(w * PN * RB + pn * RB + rb) * 64 + lane] = acc[pn][rb];
    __syncthreads();
    for (int blk = w; blk < PN * RB; blk += a.kw) {
        f32x4 s = red[blk * 64 + lane];
        for (int ww = 1; ww < a.kw; ww++) s += red[(ww * PN * RB + blk) * 64 + lane];
        const int pn = blk / RB, rb = blk % RB;
        store_block<DT>(a, s, m0 + 16 * rb, 16 * (p0 + pn), lane);
    }
}

template <int FMT, int DT, int RB, int PN, int XL>
__global__ void __launch_bounds__(512) k_direct(Args a)
{
    direct_body<FMT, DT, RB, PN, XL>(a, blockIdx.x * PN, blockIdx.y * (16 * RB));
}

// ---------------------------------------------------------------------------
// Streaming tile kernel: mid and long prefill.
//
// NWM x NWN waves own a (NWM*WM) x (16*WPB*NWN) output tile; wave (wm, wn)
// owns rows [m0 + WM*wm, +WM) and panels [WPB*wn, +WPB).  Per 128-wide K
// chunk:
//   * every thread loads the raw bytes of its UPT weight runs of chunk c+1
//     and, after the chunk-c MFMAs, unpacks them into the other half of a
//     double-buffered LDS weight tile: each weight is unpacked once per
//     workgroup and shared by all NWM*WM rows;
//   * each wave loads its own activation fragments straight from global
//     memory into VGPRs (the fragments of chunk c+1 replace those of chunk c
//     as soon as their MFMAs are issued), so X never goes through LDS;
//   * weight fragments are read from LDS one MFMA step ahead of their use;
//   * one barrier per chunk.
// Inside one MFMA, lane (r, g) of step i carries k = 128c + 32i + 8g + 0..7 in
// both operands: an activation load of step i reads 64 contiguous bytes of
// each row, and one weight run (32 consecutive k) fills the four lane groups
// of one step.
// Workgroups are renumbered so that each XCD gets a contiguous range of a
// grouped tile order (below): its L2 then serves both the shared weight
// panels and the shared activation rows.
// ---------------------------------------------------------------------------
template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int XL>
__global__ void __launch_bounds__(64 * NWM * NWN) k_stream(Args a)
{
    using XA = XLay<XL>;
    constexpr int NTG = 64 * NWM * NWN;    // threads of one K group
    constexpr int PB = WPB * NWN;          // panels per tile
    constexpr int BM = WM * NWM;           // rows per tile
    constexpr int RBW = WM / 16;           // row blocks per wave
    constexpr int UPT = PB * 64 / NTG;     // weight runs per thread per chunk
    static_assert(PB * 64 % NTG == 0 && UPT >= 1, "tile and workgroup do not divide");
    __shared__ u32x4 sW[2][PB][4][64];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
    const int wm = w % NWM, wn = w / NWM;
    const int tn = (a.np + PB - 1) / PB, tm = (a.M + BM - 1) / BM;
    int mt, nt;
    tile_coords(xcd_order(blockIdx.x, gridDim.x), tm, tn, mt, nt);
    const int m0 = mt * BM + wm * WM, p0 = nt * PB;
    const int c_lo = 0, c_hi = a.K / kChunk;
    const int r16 = lane & 15, g4 = lane >> 4;

    const uint16_t *xrow[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; rb++) {
        int r = m0 + 16 * rb + r16;
        r = r < a.M ? r : a.M - 1;
        xrow[rb] = XA::row(a, r) + XA::off(8 * g4);
    }

    f32x4 acc[WPB][RBW];
#pragma unroll
    for (int pb = 0; pb < WPB; pb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++) acc[pb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this thread's weight runs: u = tid + NT*s -> panel u/64, run (u/16)%4, column u%16
    RunSrc<FMT> src[UPT];
    RunRaw<FMT> raw[UPT];
#pragma unroll
    for (int s = 0; s < UPT; s++) {
        const int u = tid + NTG * s;
        const int p = p0 + (u >> 6);
        src[s].init(a, p < a.np ? p : a.np - 1, (u >> 4) & 3, u & 15);
    }

    // prologue: chunk 0 unpacked into LDS buffer 0, chunk 1 raw in
    // registers, chunk 0 activations in registers
    u32x4 xf[RBW][4];
#pragma unroll
    for (int s = 0; s < UPT; s++) src[s].load(c_lo, raw[s]);
#pragma unroll
    for (int rb = 0; rb < RBW; rb++)
#pragma unroll
        for (int i = 0; i < 4; i++) xf[rb][i] = *(const u32x4 *)(xrow[rb] + XA::chunk(c_lo) + XA::off(32 * i));
#pragma unroll
    for (int s = 0; s < UPT; s++) {
        u32x4 f[4];
        unpack_run<FMT, DT>(raw[s], src[s], c_lo, f);
        const int pb = (tid + NTG * s) >> 6;
#pragma unroll
        for (int j = 0; j < 4; j++) sW[0][pb][src[s].g][j * 16 + src[s].col] = f[j];
    }
    const int c1 = c_lo + 1 < c_hi ? c_lo + 1 : c_hi - 1;
#pragma unroll
    for (int s = 0; s < UPT; s++) src[s].load(c1, raw[s]);
    __syncthreads();

    // Steady state, branch-free: chunk c is multiplied from LDS buffer c&1
    // while chunk c+1 (raw bytes in registers since the start of chunk c-1)
    // is unpacked word by word into the other buffer, and the activations
    // of chunk c+1 replace those of chunk c step by step.  The raw bytes of
    // chunk c+2 are requested first, into the second register set, so a
    // whole chunk of MFMAs covers their latency.  Past the last chunk the
    // indices are clamped: the extra work is harmless (the buffer written is
    // never read again).
    RunRaw<FMT> raw2[UPT];
    auto chunk = [&](int c, int buf, RunRaw<FMT>(&ru)[UPT], RunRaw<FMT>(&rf)[UPT]) {
        const int cn = c + 1 < c_hi ? c + 1 : c_hi - 1;
        const int cnn = c + 2 < c_hi ? c + 2 : c_hi - 1;
#pragma unroll
        for (int s = 0; s < UPT; s++) src[s].load(cnn, rf[s]);
        u32x4 wcur[WPB], wnxt[WPB];
#pragma unroll
        for (int pb = 0; pb < WPB; pb++) wcur[pb] = sW[buf][wn * WPB + pb][0][lane];
        // keep the raw loads and the first LDS reads ahead of everything else
        // (left alone, the compiler sinks the loads to the end of the chunk)
        __builtin_amdgcn_sched_barrier(0);
        RunParams pr[UPT];
#pragma unroll
        for (int s = 0; s < UPT; s++) pr[s] = run_params<FMT, DT>(ru[s], src[s], cn);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (i < 3) {
#pragma unroll
                for (int pb = 0; pb < WPB; pb++) wnxt[pb] = sW[buf][wn * WPB + pb][i + 1][lane];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < RBW; rb++) {
#pragma unroll
                for (int pb = 0; pb < WPB; pb++) acc[pb][rb] = mma<DT>(wcur[pb], xf[rb][i], acc[pb][rb]);
                xf[rb][i] = *(const u32x4 *)(xrow[rb] + XA::chunk(cn) + XA::off(32 * i));
            }
#pragma unroll
            for (int s = 0; s < UPT; s++) {
                const int pb = (tid + NTG * s) >> 6;
                sW[buf ^ 1][pb][src[s].g][i * 16 + src[s].col] = unpack_word<FMT, DT>(ru[s], pr[s], i);
            }
            if (i < 3) {
#pragma unroll
                for (int pb = 0; pb < WPB; pb++) wcur[pb] = wnxt[pb];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FMT == FMT_Q4K && DT == DT_BF16) {
            // rare: runs whose d and dmin are too far apart for binary32 are
            // redone exactly (the fast words above are overwritten)
#pragma unroll
            for (int s = 0; s < UPT; s++) {
                if (pr[s].exact) {
                    const int pb = (tid + NTG * s) >> 6;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        sW[buf ^ 1][pb][src[s].g][i * 16 + src[s].col] =
                            unpack_word_exact<DT>(ru[s].codes, pr[s].fa, pr[s].nb, i);
                }
            }
        }
        __syncthreads();
    };
    int c = c_lo;
    for (; c + 1 < c_hi; c += 2) {
        chunk(c, 0, raw, raw2);
        chunk(c + 1, 1, raw2, raw);
    }
    if (c < c_hi) chunk(c, 0, raw, raw2);
#pragma unroll
    for (int pb = 0; pb < WPB; pb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
            store_block<DT>(a, acc[pb][rb], m0 + 16 * rb, 16 * (p0 + wn * WPB + pb), lane);
}

// ---------------------------------------------------------------------------
// Streaming tile kernel on 32x32x16 MFMAs.
//
// Same structure as k_stream: NWM x NWN waves (times KS K groups) own a
// (NWM*WM) x (16*WPB*NWN) tile; each weight is unpacked once per workgroup
// into a double-buffered LDS tile, activations go straight to VGPRs, one
// barrier per 128-wide chunk.  One MFMA covers 32 columns (two panels) and
// 16 K; lane (r, h) of k-step s carries k = 128c + 16s + 8h + 0..7 in both
// operands, so word i of the run g of a column lands in k-step 2g + i/2,
// lane half i%2, and an activation fragment is 16 contiguous bytes of a row.
// A wave's activation fragments sit in a ring of D k-steps (D = 8: the whole
// next chunk, for 32-row waves; fewer for the 64- and 96-row waves, whose
// accumulators leave no room for a chunk of them).
// ---------------------------------------------------------------------------
// One workgroup's pass over K chunks [c_lo, c_hi) of one tile: wave (wm, wn)
// adds its WM x (16*WPB) block of X[rows m0..][:] * W[:][panels p0..] into acc.
template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int XL, int D = 8, int LA = 1>
struct Stream32 {
    using XA = XLay<XL>;
    static constexpr int NTG = 64 * NWM * NWN;  // threads of one K group
    static constexpr int PB = WPB * NWN;        // panels per tile
    static constexpr int CB = PB / 2;           // 32-column blocks per tile
    static constexpr int CBW = WPB / 2;         // 32-column blocks per wave
    static constexpr int BM = WM * NWM;         // rows per tile
    static constexpr int RBW = WM / 32;         // 32-row blocks per wave
    static constexpr int RUNS = PB * 64;        // 32-code weight runs per chunk
    static constexpr int UPT = (RUNS + NTG - 1) / NTG;  // runs per thread per chunk
    static constexpr int UFULL = RUNS / NTG;    // slots every thread fills
    static_assert(WPB % 2 == 0 && WM % 32 == 0, "32x32 blocks");
    static_assert(UPT >= 1 && (RUNS - UFULL * NTG) % 64 == 0, "a partial slot must cover whole waves");
    typedef u32x4 Lds[2][CB][8][64];

    static __device__ __forceinline__ void run(const Args &a, Lds &sW, int tid, int lane, int wn, int m0, int p0,
                                               int c_lo, int c_hi, f32x16 (&acc)[CBW][RBW])
    {
    const uint16_t *xrow[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; rb++) {
        int r = m0 + 32 * rb + (lane & 31);
        r = r < a.M ? r : a.M - 1;
        xrow[rb] = XA::row(a, r) + XA::off(8 * (lane >> 5));
    }

    // activation fragments in flight: a ring of D k-steps (k-step s in slot
    // s % D); D = 8 holds a whole chunk ahead
    static_assert(D == 1 || D == 2 || D == 4 || D == 8, "the ring divides a chunk's eight k-steps");
    u32x4 xr[D][RBW];
    RunSrc<FMT> src[UPT];
    RunRaw<FMT> raw[UPT];
    int slot_cp[UPT], slot_lane[UPT];
#pragma unroll
    for (int s = 0; s < UPT; s++) {
        // the last slot may exist only for the first waves (every slot, when
        // a tile has fewer runs than threads); the others shadow a real run
        // (loads stay in bounds) and never store it
        const int u0 = tid + NTG * s, u = u0 < RUNS ? u0 : u0 % RUNS, pl = u >> 6, col = u & 15;
        const int p = p0 + pl;
        src[s].init(a, p < a.np ? p : a.np - 1, (u >> 4) & 3, col);
        slot_cp[s] = pl >> 1;
        slot_lane[s] = 16 * (pl & 1) + col;
    }
    // the partial slot is live for whole waves (a wave-uniform test)
    const bool extra = __builtin_amdgcn_readfirstlane(tid >> 6) < (RUNS - UFULL * NTG) / 64;
    auto live = [&](int s) { return s < UFULL || extra; };
    // word i of run g goes to k-step 2g + i/2, lane (i%2)*32 + slot_lane
    auto put = [&](int buf, int s, int i, u32x4 v) {
        if (live(s)) sW[buf][slot_cp[s]][2 * src[s].g + (i >> 1)][(i & 1) * 32 + slot_lane[s]] = v;
    };

#pragma unroll
    for (int s = 0; s < UPT; s++) src[s].load(c_lo, raw[s]);
#pragma unroll
    for (int rb = 0; rb < RBW; rb++)
#pragma unroll
        for (int ks = 0; ks < D; ks++) xr[ks][rb] = *(const u32x4 *)(xrow[rb] + XA::chunk(c_lo) + XA::off(16 * ks));
#pragma unroll
    for (int s = 0; s < UPT; s++) {
        u32x4 f[4];
        unpack_run<FMT, DT>(raw[s], src[s], c_lo, f);
#pragma unroll
        for (int i = 0; i < 4; i++) put(0, s, i, f[i]);
    }
    const int c1 = c_lo + 1 < c_hi ? c_lo + 1 : c_hi - 1;
#pragma unroll
    for (int s = 0; s < UPT; s++) src[s].load(c1, raw[s]);
    __syncthreads();

    // One chunk: MFMAs over LDS buffer `buf`, unpack of chunk c+1 (held in
    // `ru`) into the other buffer, and the raw loads of chunk c+2 into `rf`,
    // issued first so that a whole chunk of MFMAs covers their latency.  As
    // soon as the MFMAs of k-step ks are issued, its ring slot is refilled
    // with k-step ks + D (of chunk c+1 past the chunk's end).  Scheduling
    // barriers keep the compiler from sinking those loads to the end of the
    // loop and (LA = 1) put each k-step's LDS reads ahead of the previous
    // k-step's MFMAs; with LA = 0 a k-step reads its weight fragments right
    // before its MFMAs (fewer registers).
    RunRaw<FMT> raw2[UPT];
    auto chunk = [&](int c, int buf, RunRaw<FMT>(&ru)[UPT], RunRaw<FMT>(&rf)[UPT]) {
        const int cn = c + 1 < c_hi ? c + 1 : c_hi - 1;
        const int cnn = c + 2 < c_hi ? c + 2 : c_hi - 1;
#pragma unroll
        for (int s = 0; s < UPT; s++) src[s].load(cnn, rf[s]);
        u32x4 wcur[CBW], wnxt[LA ? CBW : 1];
#pragma unroll
        for (int cb = 0; cb < CBW; cb++) wcur[cb] = sW[buf][wn * CBW + cb][0][lane];
        __builtin_amdgcn_sched_barrier(0);
        RunParams pr[UPT];
#pragma unroll
        for (int s = 0; s < UPT; s++) pr[s] = run_params<FMT, DT>(ru[s], src[s], cn);
#pragma unroll
        for (int ks = 0; ks < 8; ks++) {
            if (LA && ks < 7) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wnxt[LA ? cb : 0] = sW[buf][wn * CBW + cb][ks + 1][lane];
            } else if (!LA && ks > 0) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wcur[cb] = sW[buf][wn * CBW + cb][ks][lane];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < RBW; rb++) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) acc[cb][rb] = mma32<DT>(wcur[cb], xr[ks % D][rb], acc[cb][rb]);
                xr[ks % D][rb] = *(const u32x4 *)(xrow[rb] + XA::chunk(ks + D >= 8 ? cn : c) + XA::off(16 * ((ks + D) % 8)));
            }
            if ((ks & 1) == 0) {
#pragma unroll
                for (int s = 0; s < UPT; s++) put(buf ^ 1, s, ks >> 1, unpack_word<FMT, DT>(ru[s], pr[s], ks >> 1));
            }
            if (LA && ks < 7) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wcur[cb] = wnxt[LA ? cb : 0];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FMT == FMT_Q4K && DT == DT_BF16) {
            // bf16 runs whose values may not fit binary32, redone exactly
#pragma unroll
            for (int s = 0; s < UPT; s++) {
                if (pr[s].exact) {
#pragma unroll
                    for (int i = 0; i < 4; i++) put(buf ^ 1, s, i, unpack_word_exact<DT>(ru[s].codes, pr[s].fa, pr[s].nb, i));
                }
            }
        }
        __syncthreads();
    };
    int c = c_lo;
    for (; c + 1 < c_hi; c += 2) {
        chunk(c, 0, raw, raw2);
        chunk(c + 1, 1, raw2, raw);
    }
    if (c < c_hi) chunk(c, 0, raw, raw2);
    }
};

template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS, int XL, int D = 8, int LA = 1>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_stream32(Args a)
{
    using S = Stream32<FMT, DT, WM, WPB, NWM, NWN, XL, D, LA>;
    constexpr int CBW = S::CBW, RBW = S::RBW, PB = S::PB, BM = S::BM;
    // f32x16 partial sums one K group hands over: one per (wave, block, lane)
    constexpr int NACC = NWM * NWN * CBW * RBW * 64;
    // the partial sums of groups 1.. overlay the LDS of every group (free
    // once all groups have passed their last chunk's barrier)
    static_assert(KS == 1 || (KS - 1) * NACC * sizeof(f32x16) <= KS * sizeof(typename S::Lds),
                  "K-split reduction must fit in LDS");
    __shared__ typename S::Lds sWall[KS];

    const int lane = threadIdx.x & 63, wall = threadIdx.x >> 6;
    const int kg = wall / (NWM * NWN);
    const int w = wall % (NWM * NWN), tid = threadIdx.x % S::NTG;
    const int wm = w % NWM, wn = w / NWM;
    const int tn = (a.np + PB - 1) / PB, tm = (a.M + BM - 1) / BM;
    int mt, nt;
    tile_coords(xcd_order(blockIdx.x, gridDim.x), tm, tn, mt, nt);
    const int m0 = mt * BM + wm * WM, p0 = nt * PB;
    const int nchk = a.K / kChunk / KS, c_lo = kg * nchk, c_hi = c_lo + nchk;

    f32x16 acc[CBW][RBW];
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[cb][rb][e] = 0.f;
    S::run(a, sWall[kg], tid, lane, wn, m0, p0, c_lo, c_hi, acc);
    if constexpr (KS > 1) {
        // K groups 1..KS-1 hand their partial sums to group 0 through LDS
        // (all of it is free once every group has passed its last chunk's
        // barrier); group 0 adds them in group order, independent of timing.
        f32x16 *red = reinterpret_cast<f32x16 *>(&sWall[0]);
        if (kg > 0) {
#pragma unroll
            for (int cb = 0; cb < CBW; cb++)
#pragma unroll
                for (int rb = 0; rb < RBW; rb++)
                    red[(kg - 1) * NACC + ((w * CBW + cb) * RBW + rb) * 64 + lane] = acc[cb][rb];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int g = 1; g < KS; g++)
#pragma unroll
            for (int cb = 0; cb < CBW; cb++)
#pragma unroll
                for (int rb = 0; rb < RBW; rb++)
                    acc[cb][rb] += red[(g - 1) * NACC + ((w * CBW + cb) * RBW + rb) * 64 + lane];
    }
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
            store_block32<DT>(a, acc[cb][rb], m0 + 32 * rb, 16 * p0 + 32 * (wn * CBW + cb), lane);
}

// ---------------------------------------------------------------------------
// Grouped per-expert GEMM: rows offs[e] .. offs[e+1]-1 of X and Y use expert
// e's weights (expert e's packed bytes start at W + e*wstride).  Offsets are
// clamped into [0, T] and made non-decreasing, so no access leaves X, Y or W
// whatever they hold.  Each workgroup owns one row tile of one expert: the
// grid carries an upper bound on the experts' row tiles (ceil(T/R) + E
// slots for R-row tiles), a workgroup finds its expert and tile with
// find_group_tile, and the ones past the last tile leave at once, before any
// barrier.  Two kernels:
//   * k_direct_grouped: the direct kernel's body on 16*RB rows x 4 panels,
//     K split across the waves of a workgroup when the grid is small;
//   * k_grouped_shared: 16*RB rows x 8 panels, four waves sharing each
//     chunk of activation fragments through LDS (each weight unpacked once
//     per row tile, each activation fragment fetched once per 128 columns).
// Both take row-major or fragment-major X (the fragment-major copy of the T
// routed rows; a tile's rows may start anywhere inside a 32-row block, each
// lane addresses its own row).
// ---------------------------------------------------------------------------
// Row tile j of the grouped problem: expert e, rows [lo, hi) of the expert
// (offsets clamped as k_direct_grouped clamps them), tile t of it; false
// when j is past the last tile.  The clamped bounds are prefix maxima,
// lo_e = min(M, max(0, offs[0..e])) and hi_e = lo_{e+1}, so one wave settles
// 64 experts per step with a max scan and a sum scan over its lanes; the
// result is the same in every lane.
__device__ __forceinline__ bool find_group_tile(const Args &a, int j, int BMt, int lane, int &e_out, int &lo_out,
                                                int &hi_out, int &t_out)
{
    int qc = max(0, a.offs[0]);  // max(0, offs[0..e0])
    int base = 0;
    for (int e0 = 0; e0 < a.E; e0 += 64) {
        const int e = e0 + lane;
        const bool live = e < a.E;
        int q = live ? a.offs[e + 1] : INT_MIN;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(q, d, 64);
            if (lane >= d) q = max(q, u);
        }
        q = max(q, qc);                                  // max(0, offs[0..e+1])
        int qprev = __shfl_up(q, 1, 64);
        if (lane == 0) qprev = qc;                       // max(0, offs[0..e])
        const int lo = min(qprev, a.M), hi = min(q, a.M);
        const int nb = live ? (hi - lo + BMt - 1) / BMt : 0;
        int incl = nb;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d, 64);
            if (lane >= d) incl += u;
        }
        const unsigned long long hit = __ballot(live && j < base + incl);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            e_out = e0 + l;
            lo_out = __shfl(lo, l, 64);
            hi_out = __shfl(hi, l, 64);
            t_out = j - (base + __shfl(incl, l, 64) - __shfl(nb, l, 64));
            return true;
        }
        base += __shfl(incl, 63, 64);
        qc = __shfl(q, 63, 64);
    }
    return false;
}

// Grid: x = panel groups of PN panels, y = row-tile slots of 16*RB rows.
template <int FMT, int DT, int RB, int PN, int XL>
__global__ void __launch_bounds__(512) k_direct_grouped(Args a)
{
    constexpr int R = 16 * RB;
    int e, lo, hi, t;
    // the same answer in every wave: the whole workgroup leaves together
    if (!find_group_tile(a, blockIdx.y, R, threadIdx.x & 63, e, lo, hi, t)) return;
    Args b = a;
    b.W = a.W + (long long)e * a.wstride;
    b.M = hi;
    direct_body<FMT, DT, RB, PN, XL>(b, blockIdx.x * PN, lo + t * R);
}

// Grid: x = panel groups of PN*NW panels, y = row-tile slots of 16*RB rows.
// The NW waves of a workgroup own PN panels each, side by side, over the same
// 16*RB rows of one expert.  Per chunk the workgroup copies the activation
// fragments of its rows into LDS once (each thread one or a few 16-byte
// pieces, stored in the order the lanes read them) and every wave multiplies
// them with its own weight runs, unpacked into VGPRs as in the direct kernel;
// chunk c+1's pieces wait in VGPRs while chunk c is multiplied, and one
// barrier per chunk separates the two LDS buffers.  An activation fragment
// is thus fetched once per PN*NW panels instead of once per PN, which is what
// holds the direct kernel back from tens of rows per expert on.  Each
// output's MFMAs run in the direct kernel's order, so the two give the same
// bits.
template <int FMT, int DT, int RB, int PN, int NW, int XL>
__global__ void __launch_bounds__(64 * NW) k_grouped_shared(Args a)
{
    using XA = XLay<XL>;
    constexpr int R = 16 * RB;
    constexpr int PIECES = RB * 4 * 64;                       // 16-byte pieces per chunk
    constexpr int PT = (PIECES + 64 * NW - 1) / (64 * NW);    // pieces per thread
    __shared__ u32x4 xs[2][RB][4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int e, lo, hi, t;
    // the same answer in every wave: the whole workgroup leaves together,
    // before any barrier
    if (!find_group_tile(a, blockIdx.y, R, lane, e, lo, hi, t)) return;
    Args b = a;
    b.W = a.W + (long long)e * a.wstride;
    b.M = hi;
    const int m0 = lo + t * R;
    const int p0 = (blockIdx.x * NW + w) * PN;
    const int col = lane & 15, g = lane >> 4;
    const int nch = a.K / kChunk;

    // piece q: row block q/256, fragment (q/64)%4 of lane q%64, i.e. row
    // m0 + 16*(q/256) + q%16 (clamped: computed and discarded), columns
    // 32*((q%64)/16) + 8*((q/64)%4) .. +7 of the chunk
    const uint16_t *psrc[PT];
    int pdst[PT];
#pragma unroll
    for (int s = 0; s < PT; s++) {
        const int q = threadIdx.x + 64 * NW * s;
        const int qq = q < PIECES ? q : 0;
        pdst[s] = q < PIECES ? q : -1;
        int r = m0 + 16 * (qq >> 8) + (qq & 15);
        r = r < hi ? r : hi - 1;
        psrc[s] = XA::row(b, r) + XA::off(32 * ((qq & 63) >> 4)) + XA::off(8 * ((qq >> 6) & 3));
    }
    u32x4 *xflat = &xs[0][0][0][0];

    f32x4 acc[PN][RB];
#pragma unroll
    for (int pn = 0; pn < PN; pn++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++) acc[pn][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    RunSrc<FMT> src[PN];
#pragma unroll
    for (int pn = 0; pn < PN; pn++) {
        const int p = p0 + pn;
        src[pn].init(b, p < b.np ? p : b.np - 1, g, col);
    }

    RunRaw<FMT> raw[PN];
    u32x4 xp[PT];
#pragma unroll
    for (int s = 0; s < PT; s++) xp[s] = *(const u32x4 *)(psrc[s] + XA::chunk(0));
#pragma unroll
    for (int pn = 0; pn < PN; pn++) src[pn].load(0, raw[pn]);
#pragma unroll
    for (int s = 0; s < PT; s++)
        if (pdst[s] >= 0) xflat[pdst[s]] = xp[s];
    __syncthreads();
    for (int c = 0; c < nch; c++) {
        const int buf = c & 1;
        u32x4 wf[PN][4];
#pragma unroll
        for (int pn = 0; pn < PN; pn++) unpack_run<FMT, DT>(raw[pn], src[pn], c, wf[pn]);
        if (c + 1 < nch) {
#pragma unroll
            for (int pn = 0; pn < PN; pn++) src[pn].load(c + 1, raw[pn]);
#pragma unroll
            for (int s = 0; s < PT; s++) xp[s] = *(const u32x4 *)(psrc[s] + XA::chunk(c + 1));
        }
#pragma unroll
        for (int rb = 0; rb < RB; rb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const u32x4 xc = xs[buf][rb][i][lane];
#pragma unroll
                for (int pn = 0; pn < PN; pn++) acc[pn][rb] = mma<DT>(wf[pn][i], xc, acc[pn][rb]);
            }
        if (c + 1 < nch) {
#pragma unroll
            for (int s = 0; s < PT; s++)
                if (pdst[s] >= 0) xflat[(buf ^ 1) * PIECES + pdst[s]] = xp[s];
        }
        __syncthreads();
    }
#pragma unroll
    for (int pn = 0; pn < PN; pn++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++) store_block<DT>(b, acc[pn][rb], m0 + 16 * rb, 16 * (p0 + pn), lane);
}

// ---------------------------------------------------------------------------
// K split across workgroups, for the weight-stream regime (M of one or two
// 32-row blocks).  There every workgroup of k_stream32 reads the activations
// of its rows over all of K, so each CU pulls M*K*2 bytes of X through its
// L1 while its share of the weights is small; slice s of S instead covers
// chunks [s*C/S, (s+1)*C/S) of its tile (C = K/128), split again over the
// KS K groups inside the workgroup and reduced through LDS as in k_stream32,
// and writes its fp32 partial sums to a.part + s*a.pstride (row-major
// [M][N], rows below M).  k_splitk_reduce then adds the S slices in slice
// order and rounds once, so the result does not depend on timing.  Grid: S
// times the tiles; consecutive logical indices share a slice, so the tiles
// running together on one XCD read the same activation slice.  The same
// kernel with 96-row waves (768x64 tiles, a two-deep activation ring) serves
// a few hundred rows over a long K, where 64 column tiles times S slices fill
// the CUs in one round and each weight is unpacked once for all the rows.
// ---------------------------------------------------------------------------
template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS, int XL, int D = 8, int LA = 1>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_stream32_sk(Args a)
{
    const int S = a.split;
    using St = Stream32<FMT, DT, WM, WPB, NWM, NWN, XL, D, LA>;
    constexpr int CBW = St::CBW, RBW = St::RBW, PB = St::PB, BM = St::BM;
    constexpr int NACC = NWM * NWN * CBW * RBW * 64;
    static_assert(KS == 1 || (KS - 1) * NACC * sizeof(f32x16) <= KS * sizeof(typename St::Lds),
                  "K-split reduction must fit in LDS");
    __shared__ typename St::Lds sWall[KS];

    const int lane = threadIdx.x & 63, wall = threadIdx.x >> 6;
    const int kg = wall / (NWM * NWN);
    const int w = wall % (NWM * NWN), tid = threadIdx.x % St::NTG;
    const int wm = w % NWM, wn = w / NWM;
    const int tn = (a.np + PB - 1) / PB, tm = (a.M + BM - 1) / BM, tiles = tm * tn;
    const int L = xcd_order(blockIdx.x, gridDim.x), slice = L / tiles;
    int mt, nt;
    tile_coords(L - slice * tiles, tm, tn, mt, nt);
    const int m0 = mt * BM + wm * WM, p0 = nt * PB;
    const int nall = a.K / kChunk, s_lo = (int)((long long)slice * nall / S);
    const int nchk = ((int)((long long)(slice + 1) * nall / S) - s_lo) / KS;
    const int c_lo = s_lo + kg * nchk, c_hi = c_lo + nchk;

    f32x16 acc[CBW][RBW];
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[cb][rb][e] = 0.f;
    St::run(a, sWall[kg], tid, lane, wn, m0, p0, c_lo, c_hi, acc);
    if constexpr (KS > 1) {
        f32x16 *red = reinterpret_cast<f32x16 *>(&sWall[0]);
        if (kg > 0) {
#pragma unroll
            for (int cb = 0; cb < CBW; cb++)
#pragma unroll
                for (int rb = 0; rb < RBW; rb++)
                    red[(kg - 1) * NACC + ((w * CBW + cb) * RBW + rb) * 64 + lane] = acc[cb][rb];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int g = 1; g < KS; g++)
#pragma unroll
            for (int cb = 0; cb < CBW; cb++)
#pragma unroll
                for (int rb = 0; rb < RBW; rb++)
                    acc[cb][rb] += red[(g - 1) * NACC + ((w * CBW + cb) * RBW + rb) * 64 + lane];
    }
    float *P = a.part + (long long)slice * a.pstride;
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
            store_block32_f32(P, a.M, a.N, acc[cb][rb], m0 + 32 * rb, 16 * p0 + 32 * (wn * CBW + cb), lane);
}

// Y[i] = RN_t(sum over s = 0..S-1, in that order, of part[s*slice_stride + i])
// for the MN outputs of Y (row-major [M][N]); four outputs per thread
// (slice_stride is a multiple of 4, so every slice stays 16-byte aligned).
template <int DT>
__global__ void __launch_bounds__(256) k_splitk_reduce(const float *part, uint16_t *Y, long long MN,
                                                       long long slice_stride, int S)
{
    const long long i = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
    if (i >= MN) return;
    f32x4 v = *(const f32x4 *)(part + i);
    for (int s = 1; s < S; s++) v += *(const f32x4 *)(part + (long long)s * slice_stride + i);
    const uint32_t lo = pack_out<DT>(v[0], v[1]), hi = pack_out<DT>(v[2], v[3]);
    if (i + 4 <= MN) {
        *(u32x2 *)(Y + i) = u32x2{lo, hi};
    } else {
        const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
        for (int j = 0; i + j < MN; j++) Y[i + j] = e[j];
    }
}

template <int FMT, int DT, int RB, int PN, int XL>
hipError_t launch_direct_rp(const Plan &pl, const Args &a, hipStream_t s)
{
    hipLaunchKernelGGL((k_direct<FMT, DT, RB, PN, XL>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    return hipGetLastError();
}

template <int FMT, int DT, int XL>
hipError_t launch_direct(const Plan &pl, const Args &a, hipStream_t s)
{
    if (pl.pn == 1) {
        switch (pl.rb) {
        case 1: return launch_direct_rp<FMT, DT, 1, 1, XL>(pl, a, s);
        case 2: return launch_direct_rp<FMT, DT, 2, 1, XL>(pl, a, s);
        case 3: return launch_direct_rp<FMT, DT, 3, 1, XL>(pl, a, s);
        default: return launch_direct_rp<FMT, DT, 4, 1, XL>(pl, a, s);
        }
    }
    if (pl.rb > 1)
        return pl.rb == 2 ? launch_direct_rp<FMT, DT, 2, 4, XL>(pl, a, s) : launch_direct_rp<FMT, DT, 3, 4, XL>(pl, a, s);
    switch (pl.pn) {
    case 2: return launch_direct_rp<FMT, DT, 1, 2, XL>(pl, a, s);
    case 3: return launch_direct_rp<FMT, DT, 1, 3, XL>(pl, a, s);
    default: return launch_direct_rp<FMT, DT, 1, 4, XL>(pl, a, s);
    }
}

template <int FMT, int DT, int XL>
hipError_t launch_fd(const Plan &pl, const Args &a, hipStream_t s)
{
    const bool even = (a.K / kChunk) % 2 == 0;  // an odd chunk count is not split
    switch (pl.rung) {
    case RUNG_M16_256:
        hipLaunchKernelGGL((k_stream<FMT, DT, 32, 8, 8, 1, XL>), pl.grid, dim3(512), 0, s, a);
        return hipGetLastError();
    case RUNG_M128:
        hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 8, 4, 1, 1, XL>), pl.grid, dim3(256), 0, s, a);
        return hipGetLastError();
    case RUNG_M128_K2:
        if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 8, 4, 1, 2, XL>), pl.grid, dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 8, 4, 1, 1, XL>), pl.grid, dim3(256), 0, s, a);
        return hipGetLastError();
    case RUNG_M128N160:
        hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 10, 4, 1, 1, XL>), pl.grid, dim3(256), 0, s, a);
        return hipGetLastError();
    case RUNG_M352N96:
        hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 6, 11, 1, 1, XL>), pl.grid, dim3(704), 0, s, a);
        return hipGetLastError();
    case RUNG_M768N96:
        hipLaunchKernelGGL((k_stream32<FMT, DT, 96, 6, 8, 1, 1, XL, 1, 1>), pl.grid, dim3(512), 0, s, a);
        return hipGetLastError();
    case RUNG_M512N128:
        hipLaunchKernelGGL((k_stream32<FMT, DT, 64, 8, 8, 1, 1, XL, 2, 1>), pl.grid, dim3(512), 0, s, a);
        return hipGetLastError();
    case RUNG_M512N96:
        hipLaunchKernelGGL((k_stream32<FMT, DT, 64, 6, 8, 1, 1, XL, 4, 1>), pl.grid, dim3(512), 0, s, a);
        return hipGetLastError();
    case RUNG_M192N96_K2:
        if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 6, 6, 1, 2, XL>), pl.grid, dim3(768), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 6, 6, 1, 1, XL>), pl.grid, dim3(384), 0, s, a);
        return hipGetLastError();
    case RUNG_M192N64_K2:
        if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 6, 1, 2, XL>), pl.grid, dim3(768), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 6, 1, 1, XL>), pl.grid, dim3(384), 0, s, a);
        return hipGetLastError();
    case RUNG_M768N64_SK:
        hipLaunchKernelGGL((k_stream32_sk<FMT, DT, 96, 4, 8, 1, 1, XL, 2, 1>), pl.grid, dim3(512), 0, s, a);
        return hipGetLastError();
    case RUNG_M64_SK:
        if (pl.kw == 4)
            hipLaunchKernelGGL((k_stream32_sk<FMT, DT, 32, 4, 2, 1, 4, XL>), pl.grid, dim3(512), 0, s, a);
        else if (pl.kw == 2)
            hipLaunchKernelGGL((k_stream32_sk<FMT, DT, 32, 4, 2, 1, 2, XL>), pl.grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32_sk<FMT, DT, 32, 4, 2, 1, 1, XL>), pl.grid, dim3(128), 0, s, a);
        return hipGetLastError();
    case RUNG_M64_K4:
        if ((a.K / kChunk) % 4 == 0)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 2, 1, 4, XL>), pl.grid, dim3(512), 0, s, a);
        else if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 2, 1, 2, XL>), pl.grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 2, 1, 1, XL>), pl.grid, dim3(128), 0, s, a);
        return hipGetLastError();
    case RUNG_M64N32_K4:
        if ((a.K / kChunk) % 4 == 0)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 2, 2, 1, 4, XL>), pl.grid, dim3(512), 0, s, a);
        else if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 2, 2, 1, 2, XL>), pl.grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 2, 2, 1, 1, XL>), pl.grid, dim3(128), 0, s, a);
        return hipGetLastError();
    case RUNG_M128N64_K2:
        if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 4, 1, 2, XL>), pl.grid, dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 4, 4, 1, 1, XL>), pl.grid, dim3(256), 0, s, a);
        return hipGetLastError();
    case RUNG_M96N32_K4:
        if ((a.K / kChunk) % 4 == 0)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 2, 3, 1, 4, XL>), pl.grid, dim3(768), 0, s, a);
        else if (even)
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 2, 3, 1, 2, XL>), pl.grid, dim3(384), 0, s, a);
        else
            hipLaunchKernelGGL((k_stream32<FMT, DT, 32, 2, 3, 1, 1, XL>), pl.grid, dim3(192), 0, s, a);
        return hipGetLastError();
    default:
        break;
    }
    return launch_direct<FMT, DT, XL>(pl, a, s);
}

}  // namespace qg
