// kernels_i8.h -- the int8-activation path: the row quantizer, the
// per-column requantization factors, the streaming int8 tiles (weights
// unpacked straight to int8 inside the GEMM) and the K split across
// workgroups with its exact epilogue.
#pragma once

#include "common.h"
#include "plan.h"

namespace qg {

// ---------------------------------------------------------------------------
// int8-activation variant.
//
// Activations are quantized per row to int8 in one pass (the row held in
// registers, as in the batched-prefill PR's row quantizer); weights go from
// their packed bytes straight to int8 inside the GEMM, requantized per output
// column with factors computed once at load; the contraction runs on
// 32x32x32 int8 MFMAs with exact int32 sums and one binary32 rescale per
// output.  Every step is defined to the bit:
//   w32 = RN_f32(exact weight)        (the same FMA as the fp16 unpack)
//   qw  = RNE(w32 * r_n), qx = RNE(x * r_m)   (one FMA with 1.5*2^23 each)
//   Y   = RN_t(RN_f32(acc) * RN_f32(s_m * s_n))
// with r = RN_f32(127/amax) and s = RN_f32(amax/127) of the column's binary32
// weights or the row's activations (both 0 when amax < 2^-96, which only a
// bf16 row can reach).  The int8 activations are stored fragment-major:
// 32-row blocks, each a run of 32-wide k-steps of 1 KB in which lane (r, h)
// holds row r, k = 32s + 16h .. +15:
//   Xq[m][k] at (m/32)*32*K + (k/32)*1024 + ((k/16)%2)*512 + (m%32)*16 + k%16.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
constexpr float kRneMagic = 12582912.0f;  // 1.5 * 2^23: binary32 values in [2^23, 2^24) are the integers

// The quotients are formed in binary64 (correctly rounded) and rounded again
// to binary32: for a quotient that equals one rounding of the exact value,
// since 53 >= 2*24 + 2 (Figueroa, "When is double rounding innocuous?").
__device__ __forceinline__ void i8_scales(float amax, float &r, float &s)
{
    if (!(amax >= 0x1p-96f)) {
        r = 0.0f;
        s = 0.0f;
        return;
    }
    r = (float)(127.0 / (double)amax);
    s = (float)((double)amax / 127.0);
}

// RN(v*r + 1.5*2^23) is 1.5*2^23 + RNE(v*r) for |v*r| < 2^22 (one rounding of
// the exact product plus an integer); its low byte is RNE(v*r) in two's
// complement.  |v*r| <= 127*(1 + 2^-24) for every v of the row or column
// that gave r, so the code is never above 127.
__device__ __forceinline__ uint32_t i8_code_bits(float v, float r)
{
    return __builtin_bit_cast(uint32_t, __builtin_fmaf(v, r, kRneMagic));
}

// The low bytes of a, b, c, d as one word (byte 0 = a): three byte permutes.
// v_perm_b32 picks each result byte from the eight bytes {src1 (0..3),
// src0 (4..7)}; selector 0x0c gives a zero byte.
__device__ __forceinline__ uint32_t pack4_i8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a.0, b.0, 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);  // c.0, d.0, 0, 0
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);             // a.0, b.0, c.0, d.0
}

// Element e (0 or 1) of a pair of activations, exactly widened to binary32.
template <int DT>
__device__ __forceinline__ float x_elem(uint32_t w, int e)
{
    if constexpr (DT == DT_F16) {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        return (float)(e ? h.y : h.x);
    } else {
        return __builtin_bit_cast(float, e ? (w & 0xFFFF0000u) : (w << 16));
    }
}

template <int DT>
__device__ __forceinline__ float vec_amax(u32x4 v)
{
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) a = fmaxf(a, fabsf(x_elem<DT>(v[j >> 1], j & 1)));
    return a;
}

template <int DT>
__device__ __forceinline__ u32x2 vec_codes(u32x4 v, float r)
{
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = i8_code_bits(x_elem<DT>(v[j >> 1], j & 1), r);
    return u32x2{pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7])};
}

// Row quantizer: one wave per row of the padded 32-row blocks, four rows per
// workgroup.  Each lane keeps up to kQv 8-element vectors of its row in
// registers between the max (a wave reduction, no LDS and no barrier) and
// the code pass; rows longer than 64*8*kQv elements reread the rest (from
// L2).  Rows at or past M are written as zeros.
constexpr int kQv = 24;

template <int DT>
__global__ void __launch_bounds__(256) k_i8_quant(const uint16_t *X, uint8_t *Xq, float *sx, int M, int K)
{
    const int lane = threadIdx.x & 63, m = 4 * blockIdx.x + (threadIdx.x >> 6), nv = K >> 3;
    uint8_t *qrow = Xq + (long long)(m >> 5) * 32 * K + (m & 31) * 16;
    // the 8 codes of vector v (k = 8v .. 8v+7): one half of a lane's 16 bytes
    auto dst = [&](int v) -> u32x2 * {
        const int k = 8 * v;
        return reinterpret_cast<u32x2 *>(qrow + (long long)(k >> 5) * 1024 + ((k >> 4) & 1) * 512 + (k & 15));
    };
    if (m >= M) {
        for (int v = lane; v < nv; v += 64) *dst(v) = u32x2{0u, 0u};
        return;
    }
    const uint16_t *xr = X + (long long)m * K;
    u32x4 held[kQv];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kQv; j++) {
        const int v = lane + 64 * j;
        held[j] = u32x4{0u, 0u, 0u, 0u};
        if (v < nv) held[j] = *reinterpret_cast<const u32x4 *>(xr + 8 * v);
        amax = fmaxf(amax, vec_amax<DT>(held[j]));
    }
    for (int v = lane + 64 * kQv; v < nv; v += 64)
        amax = fmaxf(amax, vec_amax<DT>(*reinterpret_cast<const u32x4 *>(xr + 8 * v)));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    float r, s;
    i8_scales(amax, r, s);
    if (lane == 0) sx[m] = s;
#pragma unroll
    for (int j = 0; j < kQv; j++) {
        const int v = lane + 64 * j;
        if (v < nv) *dst(v) = vec_codes<DT>(held[j], r);
    }
    for (int v = lane + 64 * kQv; v < nv; v += 64) *dst(v) = vec_codes<DT>(*reinterpret_cast<const u32x4 *>(xr + 8 * v), r);
}

// The eight binary32 weights of word i of a run, in k order: the fp16
// unpack's FMA (code * factor - bias, one rounding) without the final
// rounding to 16 bits.
template <int FMT>
__device__ __forceinline__ void unpack_word_f32(const RunRaw<FMT> &u, const RunParams &pr, int i, float (&w)[8])
{
    const uint32_t x = u.codes[i], x8 = x >> 8;
    uint32_t t[4];
    float fa = pr.fa, nb = pr.nb;
    if constexpr (FMT == FMT_Q6K) {
        fa = i < 2 ? pr.fa : pr.fa1;
        nb = i < 2 ? pr.nb : pr.nb1;
        const uint32_t h = u.hi[i >> 1];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const uint32_t lpart = (p < 2 ? x : x8) & ((p & 1) ? 0x00F000F0u : 0x000F000Fu);
            const int sigma = 4 * (i & 1) + p, T = (p & 1) ? 8 : 4, sh = 2 * sigma - T;
            const uint32_t hs = sh >= 0 ? (h >> sh) : (h << (-sh));
            t[p] = lpart | (hs & (0x00030003u << T));
        }
    } else {
        t[0] = x & 0x000F000Fu;
        t[1] = x & 0x00F000F0u;
        t[2] = x8 & 0x000F000Fu;
        t[3] = x8 & 0x00F000F0u;
    }
    const float fa16 = fa * 0.0625f;
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const f16x2 h = __builtin_bit_cast(f16x2, t[p]);
        const float f = (p & 1) ? fa16 : fa;
        w[2 * p] = __builtin_fmaf((float)h.x, f, nb);
        w[2 * p + 1] = __builtin_fmaf((float)h.y, f, nb);
    }
}

// Word i of a run as eight int8 codes RNE(w32 * r).
template <int FMT>
__device__ __forceinline__ u32x2 unpack_word_i8(const RunRaw<FMT> &u, const RunParams &pr, int i, float r)
{
    float w[8];
    unpack_word_f32<FMT>(u, pr, i, w);
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = i8_code_bits(w[j], r);
    return u32x2{pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7])};
}

// Per-column requantization factors, once per weight at load: one wave per
// panel, lane (g, col) walks run g of its column through every chunk, and
// the four lane groups combine their maxima.
template <int FMT>
__global__ void __launch_bounds__(64) k_i8_colscale(Args a, float *rw, float *sw)
{
    const int p = blockIdx.x, lane = threadIdx.x, g = lane >> 4, col = lane & 15;
    RunSrc<FMT> src;
    src.init(a, p, g, col);
    RunRaw<FMT> raw;
    float amax = 0.0f;
    const int nch = a.K / kChunk;
    for (int c = 0; c < nch; c++) {
        src.load(c, raw);
        const RunParams pr = run_params<FMT, DT_F16>(raw, src, c);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float w[8];
            unpack_word_f32<FMT>(raw, pr, i, w);
#pragma unroll
            for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(w[j]));
        }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int n = 16 * p + col;
    if (g == 0 && n < a.N) {
        float r, s;
        i8_scales(amax, r, s);
        rw[n] = r;
        sw[n] = s;
    }
}

__device__ __forceinline__ i32x16 mma_i8(u32x4 a, u32x4 b, i32x16 c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                                 0);
}

// One 32x32 int32 accumulator (Y^T layout, as store_block32) rescaled and
// stored: y = RN_t(RN_f32(acc) * RN_f32(s_m * s_n)).
template <int DT>
__device__ __forceinline__ void store_block_i8(const Args &a, const i32x16 &v, int m_base, int n_base, int lane)
{
    const int m = m_base + (lane & 31);
    if (m >= a.M) return;
    const float sm = a.sx[m];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int n0 = n_base + 8 * q + 4 * (lane >> 5);
        if (n0 >= a.N) continue;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float sn = n0 + j < a.N ? a.sw[n0 + j] : 0.0f;
            y[j] = (float)v[4 * q + j] * (sm * sn);
        }
        uint16_t *yp = a.Y + (long long)m * a.N + n0;
        const uint32_t lo = pack_out<DT>(y[0], y[1]), hi = pack_out<DT>(y[2], y[3]);
        if (n0 + 4 <= a.N && (a.N & 3) == 0) {
            *(u32x2 *)yp = u32x2{lo, hi};
        } else {
            const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
            for (int j = 0; j < 4 && n0 + j < a.N; j++) yp[j] = e[j];
        }
    }
}

// Streaming int8 tile: the structure of Stream32 (W unpacked once per
// workgroup into double-buffered LDS, activations straight to VGPRs, raw
// weight bytes two chunks ahead, one barrier per 128-wide chunk) on 32x32x32
// int8 MFMAs.  A chunk is four k-steps of 32; run g of a column (32 codes)
// is k-step g, lane halves 0 (words 0, 1) and 1 (words 2, 3), so both
// operands carry k = 128c + 32s + 16h + 0..15 in lane (r, h) of k-step s.
// CPB chunks share one LDS stage and one barrier (a stage of 4*CPB k-steps;
// chunk j of a stage is k-steps 4j .. 4j+3): an int8 chunk is only four
// k-steps of MFMAs, so with CPB = 2 the barrier and the LDS round trip after
// it are paid half as often.  Each thread then unpacks one run of each chunk
// of the stage (same column and lane group).
template <int FMT, int WM, int WPB, int NWM, int NWN, int CPB, int D = 4 * CPB>
struct StreamI8 {
    static constexpr int NTG = 64 * NWM * NWN;
    static constexpr int PB = WPB * NWN;
    static constexpr int CB = PB / 2;
    static constexpr int CBW = WPB / 2;
    static constexpr int BM = WM * NWM;
    static constexpr int RBW = WM / 32;
    static constexpr int RUNS = PB * 64;
    static constexpr int UPT = (RUNS + NTG - 1) / NTG;
    static constexpr int UFULL = RUNS / NTG;
    static constexpr int KSTEPS = 4 * CPB;  // k-steps per stage
    static_assert(WPB % 2 == 0 && WM % 32 == 0, "32x32 blocks");
    static_assert(UPT >= 1 && (RUNS - UFULL * NTG) % 64 == 0, "a partial slot must cover whole waves");
    static_assert(CPB == 1 || CPB == 2, "one or two chunks per stage");
    typedef u32x4 Lds[2][CB][KSTEPS][64];

    // Stages [c_lo, c_hi) (stage t = chunks CPB*t .. CPB*t+CPB-1).
    static __device__ __forceinline__ void run(const Args &a, Lds &sW, int tid, int lane, int wn, int m0, int p0,
                                               int c_lo, int c_hi, i32x16 (&acc)[CBW][RBW])
    {
    const uint8_t *Xq = reinterpret_cast<const uint8_t *>(a.X);
    const int nblk = (a.M + 31) >> 5;
    const uint8_t *xrow[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; rb++) {
        // blocks past the last one hold no rows below M: read the last (in
        // bounds), store nothing
        const int blk = min((m0 >> 5) + rb, nblk - 1);
        xrow[rb] = Xq + (long long)blk * 32 * a.K + (lane & 31) * 16 + (lane >> 5) * 512;
    }

    // activation fragments in flight: a ring of D k-steps (k-step s in slot
    // s % D); D = KSTEPS holds a whole stage ahead
    static_assert(KSTEPS % D == 0, "the ring divides a stage's k-steps");
    u32x4 xr[D][RBW];
    RunSrc<FMT> src[UPT];
    RunRaw<FMT> raw[UPT][CPB];
    int slot_cp[UPT], slot_lane[UPT];
    float rs[UPT];
#pragma unroll
    for (int s = 0; s < UPT; s++) {
        // a slot past the tile's runs (the last slot of the later waves, or
        // every slot when a tile has fewer runs than threads) shadows a real
        // run, so its loads stay in bounds; it never stores
        const int u0 = tid + NTG * s, u = u0 < RUNS ? u0 : u0 % RUNS, pl = u >> 6, col = u & 15;
        const int p = p0 + pl, n = 16 * p + col;
        src[s].init(a, p < a.np ? p : a.np - 1, (u >> 4) & 3, col);
        slot_cp[s] = pl >> 1;
        slot_lane[s] = 16 * (pl & 1) + col;
        rs[s] = (p < a.np && n < a.N) ? a.rw[n] : 0.0f;
    }
    const bool extra = __builtin_amdgcn_readfirstlane(tid >> 6) < (RUNS - UFULL * NTG) / 64;
    auto live = [&](int s) { return s < UFULL || extra; };
    // run g of chunk j of the stage is k-step 4j + g
    auto put = [&](int buf, int s, int j, int h, u32x4 v) {
        if (live(s)) sW[buf][slot_cp[s]][4 * j + src[s].g][h * 32 + slot_lane[s]] = v;
    };
    auto xload = [&](int rb, int t, int ks) {
        return *reinterpret_cast<const u32x4 *>(xrow[rb] + (long long)t * (CPB * 4096) + ks * 1024);
    };
    auto load_stage = [&](int t, RunRaw<FMT>(&r)[UPT][CPB]) {
#pragma unroll
        for (int s = 0; s < UPT; s++)
#pragma unroll
            for (int j = 0; j < CPB; j++) src[s].load(CPB * t + j, r[s][j]);
    };

    load_stage(c_lo, raw);
#pragma unroll
    for (int rb = 0; rb < RBW; rb++)
#pragma unroll
        for (int ks = 0; ks < D; ks++) xr[ks][rb] = xload(rb, c_lo, ks);
#pragma unroll
    for (int s = 0; s < UPT; s++) {
#pragma unroll
        for (int j = 0; j < CPB; j++) {
            const RunParams pr = run_params<FMT, DT_F16>(raw[s][j], src[s], CPB * c_lo + j);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const u32x2 w0 = unpack_word_i8<FMT>(raw[s][j], pr, 2 * h, rs[s]);
                const u32x2 w1 = unpack_word_i8<FMT>(raw[s][j], pr, 2 * h + 1, rs[s]);
                put(0, s, j, h, u32x4{w0.x, w0.y, w1.x, w1.y});
            }
        }
    }
    load_stage(c_lo + 1 < c_hi ? c_lo + 1 : c_hi - 1, raw);
    __syncthreads();

    // One stage: MFMAs over LDS buffer `buf`, the unpack of stage t+1 (held
    // in `ru`, one word of each of its runs per k-step) into the other
    // buffer, and the raw loads of stage t+2 into `rf`, issued first.
    RunRaw<FMT> raw2[UPT][CPB];
    auto stage = [&](int t, int buf, RunRaw<FMT>(&ru)[UPT][CPB], RunRaw<FMT>(&rf)[UPT][CPB]) {
        const int tn = t + 1 < c_hi ? t + 1 : c_hi - 1;
        const int tnn = t + 2 < c_hi ? t + 2 : c_hi - 1;
        load_stage(tnn, rf);
        u32x4 wcur[CBW], wnxt[CBW];
#pragma unroll
        for (int cb = 0; cb < CBW; cb++) wcur[cb] = sW[buf][wn * CBW + cb][0][lane];
        __builtin_amdgcn_sched_barrier(0);
        RunParams pr[UPT][CPB];
#pragma unroll
        for (int s = 0; s < UPT; s++)
#pragma unroll
            for (int j = 0; j < CPB; j++) pr[s][j] = run_params<FMT, DT_F16>(ru[s][j], src[s], CPB * tn + j);
        u32x2 pend[UPT];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            if (ks < KSTEPS - 1) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wnxt[cb] = sW[buf][wn * CBW + cb][ks + 1][lane];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < RBW; rb++) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) acc[cb][rb] = mma_i8(wcur[cb], xr[ks % D][rb], acc[cb][rb]);
                xr[ks % D][rb] = xload(rb, ks + D >= KSTEPS ? tn : t, (ks + D) % KSTEPS);
            }
            // word ks%4 of the runs of chunk ks/4
            const int j = ks >> 2, i = ks & 3;
#pragma unroll
            for (int s = 0; s < UPT; s++) {
                const u32x2 wv = unpack_word_i8<FMT>(ru[s][j], pr[s][j], i, rs[s]);
                if (i & 1) put(buf ^ 1, s, j, i >> 1, u32x4{pend[s].x, pend[s].y, wv.x, wv.y});
                else pend[s] = wv;
            }
            if (ks < KSTEPS - 1) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wcur[cb] = wnxt[cb];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };
    int t = c_lo;
    for (; t + 1 < c_hi; t += 2) {
        stage(t, 0, raw, raw2);
        stage(t + 1, 1, raw2, raw);
    }
    if (t < c_hi) stage(t, 0, raw, raw2);
    }
};

template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS, int CPB = 1, int D = 4 * CPB>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_i8_stream(Args a)
{
    using S = StreamI8<FMT, WM, WPB, NWM, NWN, CPB, D>;
    constexpr int CBW = S::CBW, RBW = S::RBW, PB = S::PB, BM = S::BM;
    constexpr int NACC = NWM * NWN * CBW * RBW * 64;
    // the partial sums of groups 1.. overlay the LDS of every group (free
    // once all groups have passed their last stage's barrier); the array is
    // sized for whichever of the two needs more
    constexpr size_t kStageBytes = KS * sizeof(typename S::Lds);
    constexpr size_t kRedBytes = KS > 1 ? (KS - 1) * NACC * sizeof(i32x16) : 0;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kStageBytes > kRedBytes ? kStageBytes : kRedBytes];
    auto &sWall = *reinterpret_cast<typename S::Lds(*)[KS]>(smem);

    const int lane = threadIdx.x & 63, wall = threadIdx.x >> 6;
    const int kg = wall / (NWM * NWN);
    const int w = wall % (NWM * NWN), tid = threadIdx.x % S::NTG;
    const int wm = w % NWM, wn = w / NWM;
    const int tn = (a.np + PB - 1) / PB, tm = (a.M + BM - 1) / BM;
    int mt, nt;
    tile_coords(xcd_order(blockIdx.x, gridDim.x), tm, tn, mt, nt);
    const int m0 = mt * BM + wm * WM, p0 = nt * PB;
    const int nstg = a.K / (kChunk * CPB) / KS, c_lo = kg * nstg, c_hi = c_lo + nstg;

    i32x16 acc[CBW][RBW];
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[cb][rb][e] = 0;
    S::run(a, sWall[kg], tid, lane, wn, m0, p0, c_lo, c_hi, acc);
    if constexpr (KS > 1) {
        // integer partial sums: the order of the additions does not matter
        i32x16 *red = reinterpret_cast<i32x16 *>(smem);
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
            store_block_i8<DT>(a, acc[cb][rb], m0 + 32 * rb, 16 * p0 + 32 * (wn * CBW + cb), lane);
}

// K split across workgroups on the int8 path, for few tiles (M of a few
// 32-row blocks over few panels): slice s of a.split covers stages
// [s*T/S, (s+1)*T/S) of its tile (T = K/128 one-chunk stages), split again
// over the KS K groups inside the workgroup, and writes its int32 partial
// sums to (int *)a.part + s*a.pstride (row-major [M][N], rows below M).
// The sums are exact, so k_i8_splitk_reduce's total, and with it Y, equals
// the unsplit rungs' bit for bit.  Grid: a.split times the tiles, the tiles
// of one slice consecutive in the XCD order.
template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_i8_stream_sk(Args a)
{
    using S = StreamI8<FMT, WM, WPB, NWM, NWN, 1>;
    constexpr int CBW = S::CBW, RBW = S::RBW, PB = S::PB, BM = S::BM;
    constexpr int NACC = NWM * NWN * CBW * RBW * 64;
    constexpr size_t kStageBytes = KS * sizeof(typename S::Lds);
    constexpr size_t kRedBytes = KS > 1 ? (KS - 1) * NACC * sizeof(i32x16) : 0;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kStageBytes > kRedBytes ? kStageBytes : kRedBytes];
    auto &sWall = *reinterpret_cast<typename S::Lds(*)[KS]>(smem);

    const int lane = threadIdx.x & 63, wall = threadIdx.x >> 6;
    const int kg = wall / (NWM * NWN);
    const int w = wall % (NWM * NWN), tid = threadIdx.x % S::NTG;
    const int wm = w % NWM, wn = w / NWM;
    const int tn = (a.np + PB - 1) / PB, tm = (a.M + BM - 1) / BM, tiles = tm * tn;
    const int L = xcd_order(blockIdx.x, gridDim.x), slice = L / tiles;
    int mt, nt;
    tile_coords(L - slice * tiles, tm, tn, mt, nt);
    const int m0 = mt * BM + wm * WM, p0 = nt * PB;
    const int nall = a.K / kChunk, s_lo = (int)((long long)slice * nall / a.split);
    const int nstg = ((int)((long long)(slice + 1) * nall / a.split) - s_lo) / KS;
    const int c_lo = s_lo + kg * nstg, c_hi = c_lo + nstg;

    i32x16 acc[CBW][RBW];
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[cb][rb][e] = 0;
    S::run(a, sWall[kg], tid, lane, wn, m0, p0, c_lo, c_hi, acc);
    if constexpr (KS > 1) {
        i32x16 *red = reinterpret_cast<i32x16 *>(smem);
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
    int *P = reinterpret_cast<int *>(a.part) + (long long)slice * a.pstride;
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++) {
            const int m = m0 + 32 * rb + (lane & 31);
            if (m >= a.M) continue;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n0 = 16 * p0 + 32 * (wn * CBW + cb) + 8 * q + 4 * (lane >> 5);
                if (n0 >= a.N) continue;
                int *pp = P + (long long)m * a.N + n0;
                const i32x16 &v = acc[cb][rb];
                if (n0 + 4 <= a.N && (a.N & 3) == 0) {
                    *(i32x4 *)pp = i32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                } else {
                    for (int j = 0; j < 4 && n0 + j < a.N; j++) pp[j] = v[4 * q + j];
                }
            }
        }
}

// Y[m][n] = RN_t(RN_f32(acc) * RN_f32(sx[m] * sw[n])) with acc the int32 sum
// of the a.split slices' partial sums (exact in any order), as the unsplit
// epilogue computes it; four consecutive outputs per thread.
template <int DT>
__global__ void __launch_bounds__(256) k_i8_splitk_reduce(const int *part, const float *sx, const float *sw,
                                                          uint16_t *Y, int M, int N, long long stride, int S)
{
    const long long MN = (long long)M * N, i = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
    if (i >= MN) return;
    i32x4 v = *(const i32x4 *)(part + i);
    for (int s = 1; s < S; s++) v += *(const i32x4 *)(part + (long long)s * stride + i);
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const long long e = i + j < MN ? i + j : MN - 1;
        const int m = (int)(e / N), n = (int)(e - (long long)m * N);
        y[j] = (float)v[j] * (sx[m] * sw[n]);
    }
    const uint32_t lo = pack_out<DT>(y[0], y[1]), hi = pack_out<DT>(y[2], y[3]);
    if (i + 4 <= MN) {
        *(u32x2 *)(Y + i) = u32x2{lo, hi};
    } else {
        const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
        for (int j = 0; i + j < MN; j++) Y[i + j] = e[j];
    }
}

template <int FMT, int DT, int CPB>
hipError_t launch_i8_cpb(int base, const Plan &pl, const Args &a, hipStream_t s)
{
    switch (base) {
    case I8_M128:
        hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 8, 4, 1, 1, CPB>), pl.grid, dim3(256), 0, s, a);
        break;
    case I8_M256:
        hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 8, 8, 1, 1, CPB>), pl.grid, dim3(512), 0, s, a);
        break;
    case I8_M128_K2:
        if (pl.kw == 2)
            hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 8, 4, 1, 2, CPB>), pl.grid, dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 8, 4, 1, 1, CPB>), pl.grid, dim3(256), 0, s, a);
        break;
    case I8_M256N96:
        hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 6, 8, 1, 1, CPB>), pl.grid, dim3(512), 0, s, a);
        break;
    case I8_M352N96:
        hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 6, 11, 1, 1, CPB>), pl.grid, dim3(704), 0, s, a);
        break;
    case I8_M768N96:  // 96-row waves: one chunk per stage, activations one k-step ahead
        hipLaunchKernelGGL((k_i8_stream<FMT, DT, 96, 6, 8, 1, 1, 1, 1>), pl.grid, dim3(512), 0, s, a);
        break;
    case I8_M192N96_K2:
        if (pl.kw == 2)
            hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 6, 6, 1, 2, CPB>), pl.grid, dim3(768), 0, s, a);
        else
            hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 6, 6, 1, 1, CPB>), pl.grid, dim3(384), 0, s, a);
        break;
    case I8_M192N64_K2:
        if (pl.kw == 2)
            hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 4, 6, 1, 2, CPB>), pl.grid, dim3(768), 0, s, a);
        else
            hipLaunchKernelGGL((k_i8_stream<FMT, DT, 32, 4, 6, 1, 1, CPB>), pl.grid, dim3(384), 0, s, a);
        break;
    default:
        hipLaunchKernelGGL((k_i8_stream<FMT, DT, 64, 6, 8, 1, 1, CPB>), pl.grid, dim3(512), 0, s, a);
        break;
    }
    return hipGetLastError();
}

// Two chunks per LDS stage (half the barriers; measured 3-7% faster on the
// M = 658 layer GEMMs and 2% at M >= 2048) wherever the stages of each K
// group cover its chunks exactly, i.e. the chunk count divides by 2 * (K
// groups); one otherwise, and for the combinations that measured slower
// with two (W4A16 on 256x96: 155 against 137 us at M = 2048) or spill with
// two (Q6_K on 512x96 and on 352x96, every format on 192x96 split in two).
template <int FMT, int DT>
hipError_t launch_i8_sk(const Plan &pl, const Args &a, hipStream_t s)
{
    if (pl.kw == 4)
        hipLaunchKernelGGL((k_i8_stream_sk<FMT, DT, 32, 4, 2, 1, 4>), pl.grid, dim3(512), 0, s, a);
    else if (pl.kw == 2)
        hipLaunchKernelGGL((k_i8_stream_sk<FMT, DT, 32, 4, 2, 1, 2>), pl.grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_i8_stream_sk<FMT, DT, 32, 4, 2, 1, 1>), pl.grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

template <int FMT, int DT>
hipError_t launch_i8_fd(const Plan &pl, const Args &a, hipStream_t s)
{
    if (pl.rung == I8_M64_SK) return launch_i8_sk<FMT, DT>(pl, a, s);
    const bool slower2 = (FMT == FMT_W4 && pl.rung == I8_M256N96) || pl.rung == I8_M192N96_K2 || pl.rung == I8_M768N96 ||
                         (FMT == FMT_Q6K && (pl.rung == I8_M512N96 || pl.rung == I8_M352N96));
    if (!slower2 && (a.K / kChunk) % (2 * pl.kw) == 0) return launch_i8_cpb<FMT, DT, 2>(pl.rung, pl, a, s);
    return launch_i8_cpb<FMT, DT, 1>(pl.rung, pl, a, s);
}

}  // namespace qg
