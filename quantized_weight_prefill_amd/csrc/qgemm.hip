// qgemm.hip -- fused-dequant prefill GEMM for MI355X (gfx950, CDNA4) and the
// C ABI around it (declared in include/qgemm.h).
//
//   Y[M,N] = X[M,K] . dequant(W)[K,N]
//
// The weights arrive in the panel layout written by pack.cpp: 16 output
// columns per panel, and for every (column, 32-wide K run) 16 contiguous
// bytes of 4-bit codes in "pair order".  One lane turns such a run into four
// MFMA operand fragments of eight fp16/bf16 values with no shuffles:
//
//   * the two codes of a pair are 16 bits apart, so one AND with 0x000F000F
//     (or 0x00F000F0 for the next pair, read as 16*code) leaves two fp16
//     bit patterns whose value is code * 2^-24 -- the zero-exponent variant
//     of the 0x6400|n trick of the W4A16 PR (section 1), which needs no
//     subtraction of 1024 afterwards;
//   * one mixed-precision FMA per weight (fp16 input, binary32 arithmetic,
//     v_fma_mix) forms factor*q - bias exactly as the batched-prefill post's
//     shader does ("The fix: K-parallel batched DMMV"), with factor scaled by
//     2^24 to cancel the code's scale, and rounds it to the operand type.
//
// Every product d*sc, dmin*m, d*s, s*zp is exact in binary32 and v_fma_mix
// rounds the exact a*b+c once, so an fp16 weight is RN_16(exact).  A bf16
// weight goes through a binary32 FMA result and one conversion; that is
// RN_bf16(exact) whenever the exact value fits binary32, which holds for Q6_K
// and W4A16 always and for Q4_K whenever the exponents of d and dmin differ
// by at most 3.  Other Q4_K bf16 runs take an exact two-sum path.
//
// MFMA operands are used "transposed": the weight fragment is the A operand
// and the activation fragment the B operand, so the accumulator holds Y^T and
// each lane ends with four consecutive output columns of one row (one 8-byte
// store).  The K order inside one MFMA is a free permutation as long as both
// operands agree; each kernel picks the one that lets a lane's 32-code run
// fill whole fragments:
//   * v_mfma_f32_16x16x32 (direct kernels, the 256-row streaming tile): lane
//     (r, g) of MFMA i carries k = 128*chunk + 32*g + 8*i + 0..7 (direct) or
//     128*chunk + 32*i + 8*g + 0..7 (streaming);
//   * v_mfma_f32_32x32x16 (the k_stream32 family): lane (r, h) of k-step s
//     carries k = 128*chunk + 16*s + 8*h + 0..7.
//
// Kernels: k_direct / k_direct_grouped (small M: each wave unpacks its own
// runs, waves split K), k_stream (16x16x32, 256x128 tiles) and k_stream32
// (32x32x16: 128x128, 128x160, 352x96, 192x96, 192x64 and 64x64 tiles, K
// split over wave groups where it pays) for larger M (each weight unpacked
// once per workgroup into double-buffered LDS), k_stream32_sk +
// k_splitk_reduce (64x64 tiles with K also split across workgroups, for few
// tiles), k_stream32_grouped (per-expert 64x64 tiles), k_stage (the staged
// arm's unpack pass), k_dequant (logical W[K][N]); the int8-activation path's
// k_i8_quant, k_i8_colscale, k_i8_stream and k_i8_stream_sk +
// k_i8_splitk_reduce.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <mutex>
#include <vector>

#include "qgemm.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { FMT_Q4K = QGEMM_FMT_Q4K, FMT_Q6K = QGEMM_FMT_Q6K, FMT_W4 = QGEMM_FMT_W4A16 };
// internal source: weights already unpacked into the staged arm's scratch
constexpr int FMT_DENSE = 3;
enum { DT_F16 = QGEMM_F16, DT_BF16 = QGEMM_BF16 };

constexpr int kChunk = 128;  // K per step: four 32-wide runs, one per lane group
constexpr int kCUs = 256;     // compute units of one MI355X (the ladder's occupancy model)
constexpr int kGroupM = 8;   // row tiles per group in the streaming tile order
constexpr int kQ4kRec = 2304, kQ6kRec = 3360;
constexpr float kTwo24 = 16777216.0f;

struct Args {
    const uint16_t *X;
    const uint8_t *W;
    uint16_t *Y;
    int M, N, K;
    int np;      // panels of 16 columns
    int group;   // W4A16 group size
    int has_zp;  // W4A16 asymmetric
    int kw;      // direct kernel: waves splitting K inside a workgroup
    long long w4_sreg, w4_zreg;  // W4A16 byte offsets of the scale / zero regions
    const int *offs;             // grouped: E+1 row offsets (device), rows offs[e]..offs[e+1] use expert e
    int E;                       // grouped: number of experts
    long long wstride;           // grouped: packed bytes of one expert's weights
    const float *sx;             // int8 path: per-row activation scales
    const float *rw, *sw;        // int8 path: per-column weight requantization factors and scales
    float *part;                 // K split across workgroups: fp32 partial sums, one slice after another
    long long pstride;           // elements from one slice to the next
    int split;                   // number of slices
};

// Activation layouts.  X_ROW: X[m][k] at m*K + k.  X_FRAG (fragment-major):
// 32-row blocks one after the other, each a sequence of 128-wide K chunks;
// inside a chunk, eight 16-wide k-steps of 512 elements, each two halves
// (k%16 < 8, then >= 8) of 32 rows x 8 consecutive k:
//   X[m][k] at ((m/32 * K/128 + k/128) * 8 + (k/16)%8) * 512
//              + ((k/8)%2 * 32 + m%32) * 8 + k%8.
// One 32x32x16 activation fragment (32 rows x 16 k) is then 1 KB of
// contiguous memory, and any 8 consecutive k of one row (the unit every
// kernel loads) stay 16 contiguous bytes.  Kernels address X as row(m) +
// chunk(c) + off(o): off takes the within-chunk offset o (a multiple of 8,
// below 128) and is additive over offsets whose bits do not overlap.
enum { X_ROW = 0, X_FRAG = 1 };

template <int XL>
struct XLay;

template <>
struct XLay<X_ROW> {
    static __device__ __forceinline__ const uint16_t *row(const Args &a, int m) { return a.X + (long long)m * a.K; }
    static __device__ __forceinline__ long long chunk(int c) { return (long long)kChunk * c; }
    static __device__ __forceinline__ int off(int o) { return o; }
};

template <>
struct XLay<X_FRAG> {
    static __device__ __forceinline__ const uint16_t *row(const Args &a, int m)
    {
        return a.X + (long long)(m >> 5) * 32 * a.K + (m & 31) * 8;
    }
    static __device__ __forceinline__ long long chunk(int c) { return 32LL * kChunk * c; }
    static __device__ __forceinline__ int off(int o) { return ((o >> 4) & 7) * 512 + ((o >> 3) & 1) * 256; }
};

// XCD-aware renumbering: workgroup b of n runs on XCD b % 8; give each XCD a
// contiguous range of logical indices (a bijection on [0, n)).
__device__ __forceinline__ int xcd_order(int b, int n)
{
    const int xcd = b & 7, slot = b >> 3;
    return xcd * (n >> 3) + min(xcd, n & 7) + slot;
}

// Logical tile L of a tm x tn grid.  With at most kGroupM row tiles the row
// tile varies fastest, so the tiles that share one column panel (its weights)
// run together on one XCD; with more, the column tile varies fastest, so the
// tiles running together share one activation row block, the larger per-tile
// stream.
__device__ __forceinline__ void tile_coords(int L, int tm, int tn, int &mt, int &nt)
{
    const int G = tm <= kGroupM ? tm : 1;
    const int gsize = G * tn, gid = L / gsize, first_m = gid * G;
    const int gm = min(tm - first_m, G), lin = L - gid * gsize;
    mt = first_m + lin % gm;
    nt = lin / gm;
}

// ---------------------------------------------------------------------------
// Unpack primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ float f16_to_f32(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// t holds two codes as fp16 bit patterns of value code*2^-24 each.  Returns
// the operand pair RN_t(fma(code_lo*2^-24, fa, nb)), RN_t(fma(code_hi*2^-24,
// fa, nb)), the FMA in binary32 (v_fma_mix on gfx950).
template <int DT>
__device__ __forceinline__ uint32_t dq_pair(uint32_t t, float fa, float nb);

template <>
__device__ __forceinline__ uint32_t dq_pair<DT_F16>(uint32_t t, float fa, float nb)
{
    f16x2 h = __builtin_bit_cast(f16x2, t);
    float a = __builtin_fmaf((float)h.x, fa, nb);
    float b = __builtin_fmaf((float)h.y, fa, nb);
    f16x2 r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
}

template <>
__device__ __forceinline__ uint32_t dq_pair<DT_BF16>(uint32_t t, float fa, float nb)
{
    f16x2 h = __builtin_bit_cast(f16x2, t);
    float a = __builtin_fmaf((float)h.x, fa, nb);
    float b = __builtin_fmaf((float)h.y, fa, nb);
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// bf16 weight of an exact value qs*fa + nb whose binary32 rounding may be
// inexact (Q4_K with d and dmin far apart): qs*fa and nb are exact binary32
// values, a two-sum gives the rounding error of their sum, and when the
// binary32 sum sits exactly on a bf16 midpoint the error decides the side.
__device__ __forceinline__ uint16_t exact_bf16(float qs, float fa, float nb)
{
#pragma clang fp contract(off)
    const float A = qs * fa;  // exact: at most 21 significant bits
    const float s = A + nb;
    const float bb = s - A;
    const float e = (A - (s - bb)) + (nb - bb);
    uint32_t sb = __builtin_bit_cast(uint32_t, s);
    if ((sb & 0xFFFFu) == 0x8000u && e != 0.0f) sb += ((e > 0.0f) == (s > 0.0f)) ? 1u : 0xFFFFFFFFu;
    return __builtin_bit_cast(uint16_t, (__bf16)__builtin_bit_cast(float, sb));
}

// ---------------------------------------------------------------------------
// One lane's weight run: panel p, lane group g (the g-th 32-wide K run of a
// 128-wide chunk) and column col of the panel.  RunSrc holds the addresses,
// fixed for the whole K loop; load() only issues raw loads (no arithmetic on
// loaded bytes, so nothing waits on memory until the unpack).
// ---------------------------------------------------------------------------

template <int FMT>
struct RunRaw {
    u32x4 codes;
    u32x4 hd;     // Q4_K: d|dmin and the 12 scale bytes; Q6_K: 16 int8 scales
    u32x2 hi;     // Q6_K high pairs
    uint32_t d;   // Q6_K: fp16 d; W4A16: fp16 scale (raw 16-bit load)
    uint32_t z;   // W4A16: byte holding the zero-point nibble
};

template <int FMT>
struct RunSrc {
    const uint8_t *rec;    // Q4_K/Q6_K: record (panel, super-block 0); W4A16: codes of chunk 0
    const uint8_t *sc;     // W4A16: scale of (panel, group 0, col)
    const uint8_t *zp;     // W4A16: zero byte of (panel, group 0, col) (a scale byte when symmetric)
    int g, col, gshift, has_zp;

    __device__ __forceinline__ void init(const Args &a, int p, int g_, int col_)
    {
        g = g_;
        col = col_;
        has_zp = a.has_zp;
        if constexpr (FMT == FMT_Q4K) {
            rec = a.W + (long long)p * (a.K >> 8) * kQ4kRec;
        } else if constexpr (FMT == FMT_Q6K) {
            rec = a.W + (long long)p * (a.K >> 8) * kQ6kRec;
        } else {
            rec = a.W + (long long)p * (a.K >> 7) * 1024 + (16 * g + col) * 16;
            gshift = 31 - __builtin_clz((unsigned)a.group);
            const long long gi = (long long)p * (a.K >> gshift);
            sc = a.W + a.w4_sreg + gi * 32 + 2 * col;
            zp = a.has_zp ? a.W + a.w4_zreg + gi * 8 + (col >> 1) : sc;
        }
    }

    __device__ __forceinline__ void load(int c, RunRaw<FMT> &r) const
    {
        if constexpr (FMT == FMT_Q4K) {
            const uint8_t *b = rec + (long long)(c >> 1) * kQ4kRec;
            r.hd = *(const u32x4 *)(b + 16 * col);
            r.codes = *(const u32x4 *)(b + 256 + 1024 * (c & 1) + (16 * g + col) * 16);
        } else if constexpr (FMT == FMT_Q6K) {
            const uint8_t *b = rec + (long long)(c >> 1) * kQ6kRec;
            r.d = *(const uint16_t *)(b + 2 * col);
            r.hd = *(const u32x4 *)(b + 32 + 16 * col);
            r.codes = *(const u32x4 *)(b + 288 + 1024 * (c & 1) + (16 * g + col) * 16);
            r.hi = *(const u32x2 *)(b + 2336 + 512 * (c & 1) + (16 * g + col) * 8);
        } else {
            r.codes = *(const u32x4 *)(rec + (long long)c * 1024);
            const int j = (kChunk * c + 32 * g) >> gshift;
            r.d = *(const uint16_t *)(sc + (long long)j * 32);
            r.z = *(zp + (long long)j * (has_zp ? 8 : 32));
        }
    }
};

// The staged arm's source: weights already unpacked into a scratch buffer,
// 4 KB per (panel, chunk) ordered [word i][run 16g+col][16 bytes], so that a
// wave's load (or store) of word i is one contiguous kilobyte.
template <>
struct RunRaw<FMT_DENSE> {
    u32x4 w[4];
};

template <>
struct RunSrc<FMT_DENSE> {
    const uint8_t *rec;  // run (g, col) of chunk 0 of the panel
    int g, col;

    __device__ __forceinline__ void init(const Args &a, int p, int g_, int col_)
    {
        g = g_;
        col = col_;
        rec = a.W + (long long)p * (a.K / kChunk) * 4096 + (16 * g + col) * 16;
    }

    __device__ __forceinline__ void load(int c, RunRaw<FMT_DENSE> &r) const
    {
#pragma unroll
        for (int i = 0; i < 4; i++) r.w[i] = *(const u32x4 *)(rec + (long long)c * 4096 + 1024 * i);
    }
};

// Per-run dequant constants (computed once per run, reused by its four words).
struct RunParams {
    float fa, nb;    // words 0..3 (Q6_K: words 0..1): factor*2^24 and -bias
    float fa1, nb1;  // Q6_K words 2..3
    bool exact;      // bf16 Q4_K run whose values may not fit binary32
};

template <int FMT, int DT>
__device__ __forceinline__ RunParams run_params(const RunRaw<FMT> &u, const RunSrc<FMT> &src, int c)
{
    RunParams pr{};
    const int g = src.g;
    if constexpr (FMT == FMT_DENSE) {
        (void)u;
        (void)g;
        (void)c;
    } else if constexpr (FMT == FMT_Q4K) {
        const float d = f16_to_f32(u.hd[0] & 0xFFFFu), dmin = f16_to_f32(u.hd[0] >> 16);
        const uint32_t s0 = u.hd[1], s1 = u.hd[2], s2 = u.hd[3];
        const int sh = 8 * g;
        // sub-blocks 0..3: low six bits of bytes 0..3 / 4..7; sub-blocks 4..7:
        // nibbles of bytes 8..11 plus the top two bits of bytes 0..3 / 4..7
        const uint32_t sc_lo = (s0 >> sh) & 63u, m_lo = (s1 >> sh) & 63u;
        const uint32_t sc_hi = ((s2 >> sh) & 15u) | (((s0 >> (sh + 6)) & 3u) << 4);
        const uint32_t m_hi = ((s2 >> (sh + 4)) & 15u) | (((s1 >> (sh + 6)) & 3u) << 4);
        const bool upper = (c & 1) != 0;
        const uint32_t sc = upper ? sc_hi : sc_lo, m = upper ? m_hi : m_lo;
        pr.fa = d * (float)sc * kTwo24;  // factor = d*sc, exact in binary32
        pr.nb = -(dmin * (float)m);      // bias = dmin*m, exact
        pr.exact = false;
        if constexpr (DT == DT_BF16) {
            // exponent fields of d and dmin (a subnormal counts as exponent 1)
            const int ed = max((int)((u.hd[0] >> 10) & 31u), 1), em = max((int)((u.hd[0] >> 26) & 31u), 1);
            pr.exact = sc != 0 && m != 0 && (ed - em > 3 || em - ed > 3);
        }
    } else if constexpr (FMT == FMT_Q6K) {
        const float d = f16_to_f32(u.d);
        const uint32_t w = u.hd[2 * (c & 1) + (g >> 1)];
        const int sh = 16 * (g & 1);
        const float a0 = d * (float)(int)(int8_t)((w >> sh) & 0xFFu);  // exact
        const float a1 = d * (float)(int)(int8_t)((w >> (sh + 8)) & 0xFFu);
        pr.fa = a0 * kTwo24;
        pr.nb = -32.0f * a0;
        pr.fa1 = a1 * kTwo24;
        pr.nb1 = -32.0f * a1;
    } else {
        const float s = f16_to_f32(u.d);
        const float zp = src.has_zp ? (float)((u.z >> (4 * (src.col & 1))) & 15u) : 8.0f;
        pr.fa = s * kTwo24;
        pr.nb = -(zp * s);
    }
    return pr;
}

// Word i of a run: eight weights k0+8i .. k0+8i+7, one MFMA operand fragment.
template <int FMT, int DT>
__device__ __forceinline__ u32x4 unpack_word(const RunRaw<FMT> &u, const RunParams &pr, int i)
{
    u32x4 out;
    if constexpr (FMT == FMT_DENSE) {
        (void)pr;
        return u.w[i];
    } else {
    const uint32_t x = u.codes[i], x8 = x >> 8;
    if constexpr (FMT == FMT_Q6K) {
        const float fa = i < 2 ? pr.fa : pr.fa1, nb = i < 2 ? pr.nb : pr.nb1;
        const float fa16 = fa * 0.0625f;
        const uint32_t h = u.hi[i >> 1];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const uint32_t lpart = (p < 2 ? x : x8) & ((p & 1) ? 0x00F000F0u : 0x000F000Fu);
            const int sigma = 4 * (i & 1) + p, T = (p & 1) ? 8 : 4, sh = 2 * sigma - T;
            const uint32_t hs = sh >= 0 ? (h >> sh) : (h << (-sh));
            out[p] = dq_pair<DT>(lpart | (hs & (0x00030003u << T)), (p & 1) ? fa16 : fa, nb);
        }
    } else {
        const uint32_t t[4] = {x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u};
        const float fa16 = pr.fa * 0.0625f;
#pragma unroll
        for (int p = 0; p < 4; p++) out[p] = dq_pair<DT>(t[p], (p & 1) ? fa16 : pr.fa, pr.nb);
    }
    return out;
    }
}

// Word i of a bf16 Q4_K run whose values may not fit binary32 (pr.exact).
__device__ __noinline__ u32x4 unpack_word_exact_bf16(u32x4 codes, float fa, float nb, int i)
{
    u32x4 out;
    const uint32_t x = codes[i], x8 = x >> 8;
    const uint32_t t[4] = {x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u};
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const f16x2 h = __builtin_bit_cast(f16x2, t[p]);
        const float f = (p & 1) ? fa * 0.0625f : fa;
        out[p] = (uint32_t)exact_bf16((float)h.x, f, nb) | ((uint32_t)exact_bf16((float)h.y, f, nb) << 16);
    }
    return out;
}

template <int FMT, int DT>
__device__ __forceinline__ u32x4 unpack_word_any(const RunRaw<FMT> &u, const RunParams &pr, int i)
{
    if constexpr (FMT == FMT_Q4K && DT == DT_BF16) {
        if (pr.exact) return unpack_word_exact_bf16(u.codes, pr.fa, pr.nb, i);
    }
    return unpack_word<FMT, DT>(u, pr, i);
}

template <int FMT, int DT>
__device__ __forceinline__ void unpack_run(const RunRaw<FMT> &u, const RunSrc<FMT> &src, int c, u32x4 (&out)[4])
{
    const RunParams pr = run_params<FMT, DT>(u, src, c);
#pragma unroll
    for (int i = 0; i < 4; i++) out[i] = unpack_word_any<FMT, DT>(u, pr, i);
}

template <int DT>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mma<DT_F16>(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma<DT_BF16>(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32x16 MFMA: twice the MACs of the 16x16x32 form per instruction and, on
// gfx950, twice its sustained rate.
template <int DT>
__device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mma32<DT_F16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mma32<DT_BF16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

template <int DT>
__device__ __forceinline__ uint32_t pack_out(float a, float b)
{
    if constexpr (DT == DT_F16) {
        f16x2 r = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, r);
    } else {
        bf16x2 r = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, r);
    }
}

// Store one 16x16 accumulator (Y^T layout): lane holds rows m, columns
// n0 .. n0+3 with m = m_base + lane%16, n0 = n_base + 4*(lane/16).
template <int DT>
__device__ __forceinline__ void store_block(const Args &a, f32x4 v, int m_base, int n_base, int lane)
{
    const int m = m_base + (lane & 15);
    const int n0 = n_base + 4 * (lane >> 4);
    if (m >= a.M || n0 >= a.N) return;
    uint16_t *y = a.Y + (long long)m * a.N + n0;
    const uint32_t lo = pack_out<DT>(v[0], v[1]), hi = pack_out<DT>(v[2], v[3]);
    if (n0 + 4 <= a.N && (a.N & 3) == 0) {
        *(u32x2 *)y = u32x2{lo, hi};
    } else {
        const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
        for (int j = 0; j < 4 && n0 + j < a.N; j++) y[j] = e[j];
    }
}

// Store one 32x32 accumulator (Y^T layout): lane holds row m = m_base +
// lane%32 and, for q = 0..3, columns n_base + 8q + 4*(lane/32) + 0..3.
template <int DT>
__device__ __forceinline__ void store_block32(const Args &a, const f32x16 &v, int m_base, int n_base, int lane)
{
    const int m = m_base + (lane & 31);
    if (m >= a.M) return;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int n0 = n_base + 8 * q + 4 * (lane >> 5);
        if (n0 >= a.N) continue;
        uint16_t *y = a.Y + (long long)m * a.N + n0;
        const uint32_t lo = pack_out<DT>(v[4 * q], v[4 * q + 1]), hi = pack_out<DT>(v[4 * q + 2], v[4 * q + 3]);
        if (n0 + 4 <= a.N && (a.N & 3) == 0) {
            *(u32x2 *)y = u32x2{lo, hi};
        } else {
            const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
            for (int j = 0; j < 4 && n0 + j < a.N; j++) y[j] = e[j];
        }
    }
}

// The same block as fp32 partial sums into P[m][n] (row stride N), rows
// below M only: a K slice's share of Y before the slices are added.
__device__ __forceinline__ void store_block32_f32(float *P, int M, int N, const f32x16 &v, int m_base, int n_base,
                                                  int lane)
{
    const int m = m_base + (lane & 31);
    if (m >= M) return;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int n0 = n_base + 8 * q + 4 * (lane >> 5);
        if (n0 >= N) continue;
        float *p = P + (long long)m * N + n0;
        if (n0 + 4 <= N && (N & 3) == 0) {
            *(f32x4 *)p = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        } else {
            for (int j = 0; j < 4 && n0 + j < N; j++) p[j] = v[4 * q + j];
        }
    }
}

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

// Grouped per-expert GEMM: rows offs[e] .. offs[e+1]-1 of X and Y use expert
// e's weights (expert e's packed bytes start at W + e*wstride).  grid.y is an
// upper bound on the row blocks of all experts (ceil(T/R) + E, T = a.M);
// workgroup y walks the experts' block counts to find its own, and the ones
// past the last block exit.  Offsets are clamped into [0, T] and made
// non-decreasing, so no access leaves X, Y or W whatever they hold.
template <int FMT, int DT, int RB, int PN>
__global__ void __launch_bounds__(512) k_direct_grouped(Args a)
{
    constexpr int R = 16 * RB;
    const int j = blockIdx.y;
    int base = 0, lo = 0, hi = 0, e = 0;
    for (; e < a.E; e++) {
        lo = min(max(a.offs[e], hi), a.M);
        hi = min(max(a.offs[e + 1], lo), a.M);
        const int nb = (hi - lo + R - 1) / R;
        if (j < base + nb) break;
        base += nb;
    }
    if (e >= a.E) return;  // the whole workgroup leaves together, before any barrier
    Args b = a;
    b.W = a.W + (long long)e * a.wstride;
    b.M = hi;
    direct_body<FMT, DT, RB, PN, X_ROW>(b, blockIdx.x * PN, lo + (j - base) * R);
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
                            unpack_word_exact_bf16(ru[s].codes, pr[s].fa, pr[s].nb, i);
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
// ---------------------------------------------------------------------------
// One workgroup's pass over K chunks [c_lo, c_hi) of one tile: wave (wm, wn)
// adds its WM x (16*WPB) block of X[rows m0..][:] * W[:][panels p0..] into acc.
template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int XL>
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

    u32x4 xf[RBW][8];
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
        for (int ks = 0; ks < 8; ks++) xf[rb][ks] = *(const u32x4 *)(xrow[rb] + XA::chunk(c_lo) + XA::off(16 * ks));
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
    // issued first so that a whole chunk of MFMAs covers their latency.  The
    // activation fragment of k-step ks is reloaded for chunk c+1 as soon as
    // its MFMAs are issued.  Scheduling barriers keep the compiler from
    // sinking those loads to the end of the loop and put each k-step's LDS
    // reads ahead of the previous k-step's MFMAs.
    RunRaw<FMT> raw2[UPT];
    auto chunk = [&](int c, int buf, RunRaw<FMT>(&ru)[UPT], RunRaw<FMT>(&rf)[UPT]) {
        const int cn = c + 1 < c_hi ? c + 1 : c_hi - 1;
        const int cnn = c + 2 < c_hi ? c + 2 : c_hi - 1;
#pragma unroll
        for (int s = 0; s < UPT; s++) src[s].load(cnn, rf[s]);
        u32x4 wcur[CBW], wnxt[CBW];
#pragma unroll
        for (int cb = 0; cb < CBW; cb++) wcur[cb] = sW[buf][wn * CBW + cb][0][lane];
        __builtin_amdgcn_sched_barrier(0);
        RunParams pr[UPT];
#pragma unroll
        for (int s = 0; s < UPT; s++) pr[s] = run_params<FMT, DT>(ru[s], src[s], cn);
#pragma unroll
        for (int ks = 0; ks < 8; ks++) {
            if (ks < 7) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wnxt[cb] = sW[buf][wn * CBW + cb][ks + 1][lane];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < RBW; rb++) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) acc[cb][rb] = mma32<DT>(wcur[cb], xf[rb][ks], acc[cb][rb]);
                xf[rb][ks] = *(const u32x4 *)(xrow[rb] + XA::chunk(cn) + XA::off(16 * ks));
            }
            if ((ks & 1) == 0) {
#pragma unroll
                for (int s = 0; s < UPT; s++) put(buf ^ 1, s, ks >> 1, unpack_word<FMT, DT>(ru[s], pr[s], ks >> 1));
            }
            if (ks < 7) {
#pragma unroll
                for (int cb = 0; cb < CBW; cb++) wcur[cb] = wnxt[cb];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FMT == FMT_Q4K && DT == DT_BF16) {
#pragma unroll
            for (int s = 0; s < UPT; s++) {
                if (pr[s].exact) {
#pragma unroll
                    for (int i = 0; i < 4; i++) put(buf ^ 1, s, i, unpack_word_exact_bf16(ru[s].codes, pr[s].fa, pr[s].nb, i));
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

template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS, int XL>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_stream32(Args a)
{
    using S = Stream32<FMT, DT, WM, WPB, NWM, NWN, XL>;
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
// Grouped streaming tiles (per-expert GEMM, rows pre-grouped by expert):
// each workgroup owns one 64x64 tile of one expert (two 32-row waves per K
// group, KS K groups reduced through LDS as in k_stream32), so an expert's
// activation rows are read once per 64 columns instead of once per 16 as in
// k_direct_grouped.  Grid: (ceil(T/64) + E) row-tile slots (an upper bound of
// the experts' row tiles) times the column tiles; a workgroup finds its
// expert by scanning the device offsets (clamped to be non-decreasing and at
// most T, as k_direct_grouped does) and leaves at once, before any barrier,
// when its slot is past the last tile.  Activations row-major.
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

template <int FMT, int DT, int KS>
__global__ void __launch_bounds__(128 * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_stream32_grouped(Args a)
{
    using St = Stream32<FMT, DT, 32, 4, 2, 1, X_ROW>;
    constexpr int CBW = St::CBW, RBW = St::RBW, PB = St::PB, BM = St::BM;
    constexpr int NACC = 2 * CBW * RBW * 64;
    static_assert(KS == 1 || (KS - 1) * NACC * sizeof(f32x16) <= KS * sizeof(typename St::Lds),
                  "K-split reduction must fit in LDS");
    __shared__ typename St::Lds sWall[KS];

    const int tn = (a.np + PB - 1) / PB;
    const int nt = blockIdx.x % tn, j = blockIdx.x / tn;
    const int lane = threadIdx.x & 63, wall = threadIdx.x >> 6;
    int e, lo, hi, t;
    // every wave computes the same answer: the whole workgroup leaves
    // together, before any barrier
    if (!find_group_tile(a, j, BM, lane, e, lo, hi, t)) return;
    Args b = a;
    b.W = a.W + (long long)e * a.wstride;
    b.M = hi;

    const int kg = wall / 2, w = wall % 2, tid = threadIdx.x % St::NTG;
    const int m0 = lo + t * BM + w * 32, p0 = nt * PB;
    const int nchk = a.K / kChunk / KS, c_lo = kg * nchk, c_hi = c_lo + nchk;

    f32x16 acc[CBW][RBW];
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[cb][rb][q] = 0.f;
    St::run(b, sWall[kg], tid, lane, 0, m0, p0, c_lo, c_hi, acc);
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
#pragma unroll
    for (int cb = 0; cb < CBW; cb++)
#pragma unroll
        for (int rb = 0; rb < RBW; rb++)
            store_block32<DT>(b, acc[cb][rb], m0 + 32 * rb, 16 * p0 + 32 * cb, lane);
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
// running together on one XCD read the same activation slice.
// ---------------------------------------------------------------------------
template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS, int XL>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_stream32_sk(Args a)
{
    const int S = a.split;
    using St = Stream32<FMT, DT, WM, WPB, NWM, NWN, XL>;
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

// ---------------------------------------------------------------------------
// Logical dequant: the same unpack, written out as W[K][N] (row-major).
// One thread per (panel, chunk, run, column).
// ---------------------------------------------------------------------------
template <int FMT, int DT>
__global__ void __launch_bounds__(256) k_dequant(Args a, uint16_t *Wout)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int nch = a.K / kChunk;
    const long long total = (long long)a.np * nch * 64;
    if (idx >= total) return;
    const int lane = (int)(idx & 63), col = lane & 15, g = lane >> 4;
    const long long pc = idx >> 6;
    const int c = (int)(pc % nch), p = (int)(pc / nch);
    const int n = 16 * p + col;
    RunSrc<FMT> src;
    src.init(a, p, g, col);
    RunRaw<FMT> raw;
    src.load(c, raw);
    u32x4 f[4];
    unpack_run<FMT, DT>(raw, src, c, f);
    if (n >= a.N) return;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const long long k = (long long)kChunk * c + 32 * g + 8 * i + 2 * j;
            Wout[k * a.N + n] = (uint16_t)(f[i][j] & 0xFFFFu);
            Wout[(k + 1) * a.N + n] = (uint16_t)(f[i][j] >> 16);
        }
}

// ---------------------------------------------------------------------------
// Staged arm, step one: the same unpack, written to a scratch buffer in the
// order the streaming kernel reads it (the FMT_DENSE layout): one thread per
// (panel, chunk, run); a wave's four 16-byte stores are four contiguous
// kilobytes.  Step two is k_stream32<FMT_DENSE, ...> on that scratch.
// ---------------------------------------------------------------------------
template <int FMT, int DT>
__global__ void __launch_bounds__(256) k_stage(Args a, uint8_t *Ws)
{
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int nch = a.K / kChunk;
    const long long total = (long long)a.np * nch * 64;
    if (idx >= total) return;
    const int run = (int)(idx & 63), col = run & 15, g = run >> 4;
    const long long pc = idx >> 6;  // = panel * nch + chunk
    const int c = (int)(pc % nch), p = (int)(pc / nch);
    RunSrc<FMT> src;
    src.init(a, p, g, col);
    RunRaw<FMT> raw;
    src.load(c, raw);
    u32x4 f[4];
    unpack_run<FMT, DT>(raw, src, c, f);
    u32x4 *dst = reinterpret_cast<u32x4 *>(Ws + pc * 4096) + run;
#pragma unroll
    for (int i = 0; i < 4; i++) dst[64 * i] = f[i];
}

// ---------------------------------------------------------------------------
// Fragment-major copy of X (layout X_FRAG).  One workgroup per (32-row block,
// 128-wide chunk), which is 8 KB in both layouts; each thread moves two
// 16-byte units (8 consecutive k of one row), read row-major, 16 lanes per
// row, and written to their fragment slot.  Rows at or past M become zeros.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_x_to_xf(const uint16_t *X, uint16_t *Xf, int M, int K)
{
    const int nch = K / kChunk;
    const int tile = blockIdx.x, blk = tile / nch, c = tile % nch;
    uint16_t *dst = Xf + (long long)tile * (32 * kChunk);
#pragma unroll
    for (int half = 0; half < 2; half++) {
        const int t = threadIdx.x + 256 * half;  // unit of the tile: row r, k group kq
        const int r = t >> 4, kq = t & 15;
        const int m = 32 * blk + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < M) v = *(const u32x4 *)(X + (long long)m * K + kChunk * c + 8 * kq);
        // k-step kq/2, half kq%2, row r
        *(u32x4 *)(dst + ((kq >> 1) * 64 + (kq & 1) * 32 + r) * 8) = v;
    }
}


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
template <int FMT, int WM, int WPB, int NWM, int NWN, int CPB>
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

    u32x4 xf[RBW][KSTEPS];
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
        for (int ks = 0; ks < KSTEPS; ks++) xf[rb][ks] = xload(rb, c_lo, ks);
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
                for (int cb = 0; cb < CBW; cb++) acc[cb][rb] = mma_i8(wcur[cb], xf[rb][ks], acc[cb][rb]);
                xf[rb][ks] = xload(rb, tn, ks);
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

template <int FMT, int DT, int WM, int WPB, int NWM, int NWN, int KS, int CPB = 1>
__global__ void __launch_bounds__(64 * NWM * NWN * KS) __attribute__((amdgpu_waves_per_eu(2)))
k_i8_stream(Args a)
{
    using S = StreamI8<FMT, WM, WPB, NWM, NWN, CPB>;
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

// ---------------------------------------------------------------------------
// Host side: validation, the M-ladder, launches.
// ---------------------------------------------------------------------------

enum Rung {
    RUNG_SMALL_M = 0,     // direct, one panel per wave, up to 64 rows per wave
    RUNG_SKINNY_N = 1,    // direct, up to four panels per wave, 16 rows per wave
    RUNG_WIDE = 2,        // direct, four panels and up to 48 rows per wave
    RUNG_M16_256 = 3,     // 16x16x32 MFMA: 256x128, 8 waves of 32x128
    RUNG_M128 = 4,        // 32x32x16 MFMA: 128x128, 4 waves of 32x128
    RUNG_M128_K2 = 5,     // 32x32x16 MFMA: 128x128, K split over two 4-wave groups
    RUNG_M128N160 = 6,    // 32x32x16 MFMA: 128x160, 4 waves of 32x160
    RUNG_M64_K4 = 7,      // 32x32x16 MFMA: 64x64, 2 waves of 32x64, K split over four groups
    RUNG_M352N96 = 8,     // 32x32x16 MFMA: 352x96, 11 waves of 32x96
    RUNG_M192N96_K2 = 9,  // 32x32x16 MFMA: 192x96, K split over two 6-wave groups (three waves per SIMD)
    RUNG_M192N64_K2 = 10, // 32x32x16 MFMA: 192x64, K split over two 6-wave groups
    RUNG_M64_SK = 11,     // 32x32x16 MFMA: 64x64, K split over four groups and across workgroups
    RUNG_COUNT = 12
};
const char *const kRungNames[RUNG_COUNT] = {"direct-small-m",    "direct-skinny-n",   "direct-wide",
                                            "mfma16-256x128",    "mfma32-128x128",    "mfma32-128x128-k2",
                                            "mfma32-128x160",    "mfma32-64x64-k4",   "mfma32-352x96",
                                            "mfma32-192x96-k2",  "mfma32-192x64-k2",  "mfma32-64x64-sk"};

struct Plan {
    int rung;
    int tiles_n, tiles_m;  // output tiles along N and along M
    int rows, cols;    // output tile
    int waves, kw;     // waves per workgroup, K-split ways inside one workgroup
    int split;         // K slices across workgroups (1: none)
    int rb, pn;        // direct kernel: row blocks / panels per wave
    dim3 grid;
    size_t lds;        // dynamic LDS bytes
};

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Waves splitting K inside one direct-kernel workgroup: enough waves in the
// whole grid to keep every CU streaming (about 2048), at least two chunks
// per wave, at most eight waves.  For decode-adjacent M (a pure weight
// stream) a wave keeps at least eight chunks once the grid holds 512 waves:
// with one chunk in flight ahead, shorter K ranges leave the stream idle
// while each wave starts and drains (measured at M = 1..16).
int pick_kw(long long groups, int nch, bool stream)
{
    int kw = 1;
    while (kw < 8 && groups * kw < 2048 && nch / (2 * kw) >= ((stream && groups * kw >= 512) ? 8 : 2)) kw *= 2;
    return kw;
}

// QGEMM_OK, QGEMM_ERR_FORMAT for an unknown rung, or QGEMM_ERR_SHAPE when
// the grid would exceed what one launch can address (2^31-1 workgroups
// along x, 65535 along y).
int make_plan(int rung, long long M, long long N, long long K, Plan &pl)
{
    const long long np = (N + 15) / 16;
    const int nch = (int)(K / kChunk);
    pl = Plan{};
    pl.rung = rung;
    switch (rung) {
    case RUNG_SMALL_M:
    case RUNG_SKINNY_N:
    case RUNG_WIDE: {
        if (rung == RUNG_SMALL_M) {
            pl.rb = M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : 4;
            pl.pn = 1;
        } else if (rung == RUNG_SKINNY_N) {
            pl.rb = 1;
            pl.pn = np >= 4 ? 4 : (int)np;
        } else {  // each weight run unpacked once for up to 48 rows, each activation fragment used by four panels
            pl.rb = M <= 16 ? 1 : M <= 32 ? 2 : 3;
            pl.pn = 4;
        }
        const long long gx = (np + pl.pn - 1) / pl.pn, gy = (M + 16 * pl.rb - 1) / (16 * pl.rb);
        if (gy > 65535) return QGEMM_ERR_SHAPE;
        pl.grid = dim3((unsigned)gx, (unsigned)gy, 1);
        break;
    }
    case RUNG_M16_256:
    case RUNG_M128:
    case RUNG_M128_K2:
    case RUNG_M128N160:
    case RUNG_M64_K4:
    case RUNG_M64_SK:
    case RUNG_M352N96:
    case RUNG_M192N96_K2:
    case RUNG_M192N64_K2: {
        const bool n96 = rung == RUNG_M352N96 || rung == RUNG_M192N96_K2;
        const bool r192 = rung == RUNG_M192N96_K2 || rung == RUNG_M192N64_K2;
        const bool r64 = rung == RUNG_M64_K4 || rung == RUNG_M64_SK;
        pl.rows = rung == RUNG_M16_256 ? 256 : r64 ? 64 : rung == RUNG_M352N96 ? 352 : r192 ? 192 : 128;
        pl.cols = rung == RUNG_M128N160 ? 160 : (r64 || rung == RUNG_M192N64_K2) ? 64 : n96 ? 96 : 128;
        pl.kw = ((rung == RUNG_M128_K2 || r192) && (K / kChunk) % 2 == 0) ? 2 : 1;
        if (r64) pl.kw = (K / kChunk) % 4 == 0 ? 4 : (K / kChunk) % 2 == 0 ? 2 : 1;
        pl.waves = rung == RUNG_M16_256 ? 8 : r64 ? 2 * pl.kw : rung == RUNG_M352N96 ? 11
                   : r192 ? 6 * pl.kw : 4 * pl.kw;
        // one-dimensional grid: the kernel renumbers tiles per XCD
        const long long tn = (np + pl.cols / 16 - 1) / (pl.cols / 16), tm = (M + pl.rows - 1) / pl.rows;
        if (tn * tm > INT32_MAX) return QGEMM_ERR_SHAPE;
        pl.tiles_n = (int)tn;
        pl.tiles_m = (int)tm;
        pl.split = 1;
        if (rung == RUNG_M64_SK) {
            // slices across workgroups: double while the grid stays within
            // two workgroups per CU, the slices divide the chunks evenly
            // among the in-group K groups and each group keeps four chunks
            while (pl.split < 8 && tn * tm * 2 * pl.split <= 2 * kCUs && nch % (2 * pl.split * pl.kw) == 0 &&
                   nch / (2 * pl.split * pl.kw) >= 4)
                pl.split *= 2;
        }
        if (tn * tm * pl.split > INT32_MAX) return QGEMM_ERR_SHAPE;
        pl.grid = dim3((unsigned)(tn * tm * pl.split), 1, 1);
        pl.lds = 0;
        return QGEMM_OK;
    }
    default:
        return QGEMM_ERR_FORMAT;
    }
    pl.rows = 16 * pl.rb;
    pl.cols = 16 * pl.pn;
    pl.split = 1;
    pl.tiles_n = (int)pl.grid.x;
    pl.tiles_m = (int)pl.grid.y;
    pl.kw = pick_kw((long long)pl.grid.x * pl.grid.y, nch, M <= 16);
    pl.waves = pl.kw;
    pl.lds = pl.kw > 1 ? (size_t)pl.kw * pl.pn * pl.rb * 64 * sizeof(float) * 4 : 0;
    return QGEMM_OK;
}

// The M-ladder (measured on MI355X; each rung is legal for every shape):
//  * narrow N (at most four panels): the grid must run over M, so the
//    direct kernel with all panels per wave (a 128-wide tile would leave most
//    of the part idle and most of each tile padding);
//  * decode-adjacent M (at most 64 rows): each weight feeds at most 64 rows
//    and the kernel is a weight stream; up to 16 rows one panel and all rows
//    per wave (the most waves streaming, each weight unpacked once), except
//    over 1536 panels and more and, on row-major activations, at 9..16 rows
//    over 512 panels and more: four panels and 16 rows per wave; with fewer
//    than 512 panels up to 64 rows one panel per wave, or on fragment-major
//    activations over 129..256 panels 64x64 tiles with K split across
//    workgroups too (split_pays); with many panels: 17..32 rows (17..48 for
//    Q4_K) four panels and all rows per wave (each activation fragment feeds
//    four panels), 49..64 rows of Q4_K and 33..64 of W4A16 and Q6_K 64x64
//    streaming tiles with K split four ways;
//  * fewer than 128 tiles of 128x128: the split rung where split_pays, else
//    the direct kernels, 64x64 K-split tiles or (fragment-major) 192x64
//    K-split tiles, by the round model of mid_m_rung;
//  * the 8-wave 256x128 tile on 16x16x32 MFMAs (each weight unpacked once
//    for 256 rows) when the occupancy model below has it finish no later
//    than the 128-row tiles;
//  * at most 256 tiles of 128x128 over K >= 8192: the 128x128 tile on
//    32x32x16 MFMAs with K split between two wave groups;
//  * otherwise the 128-row tile on 32x32x16 MFMAs, 128 or 160 columns wide,
//    whichever the occupancy model below finishes first.
// On fragment-major activations the three-waves-per-SIMD tiles come first
// where they fit (192x64 and 192x96 with K split over two 6-wave groups,
// 352x96; the rules are in select_rung), the K-split 128x128 tile serves the
// other shapes with at most 256 of its tiles, and the 256-row tile also wins
// whenever it has 512 tiles.
// Modeled time of a 128-row streaming rung with tiles `cols` wide, in units
// of one 128x128 tile at full CU rate: two tiles share a CU at a time, so
// the busiest of the 256 CUs carries ceil(T/256) tiles, and a tile that
// runs alone on a CU (one wave per SIMD) counts 1.43 (a constant fitted to
// the measured times of both widths at M = 300, 658 and 1024).
double stream_cost(long long M, long long np, int cols)
{
    const long long T = ((M + 127) / 128) * ((np + cols / 16 - 1) / (cols / 16));
    const long long n = (T + kCUs - 1) / kCUs;
    const double t = (n & 1) ? (double)(n - 1) + 1.43 : (double)n;
    return t * cols / 128.0;
}

// Between decode-adjacent M and 128 tiles of 128x128 three rungs compete:
// one panel and up to 64 rows per wave (direct-small-m), four panels and 48
// rows per wave (direct-wide) and 64x64 streaming tiles with K split four
// ways, and on fragment-major activations with an even chunk count a fourth,
// the 192x64 tile with K split over two 6-wave groups.  Their workgroups run
// in rounds of one per CU; a round costs a constant per rung, measured on
// MI355X with Q4_K at K = 4096 (M = 80..384, N = 1024..12288): 8, 15.5, 17
// and 27 microseconds.  The 48-row direct variant spills for Q6_K and W4A16
// and is left out for them.  (Q6_K at M = 300..384, N = 4096: 192x64 72-73
// against 91 us for the 64x64 tiles.)
// The split rung over few panels (N = 4096) on fragment-major activations:
// one panel and all rows per wave reads the activations once per panel, the
// 64x64 tiles split across workgroups read a slice of them.  Measured on
// MI355X (weights rotating):
//  * K = 12288 (four slices): Q6_K and W4A16, and every format in bf16,
//    from 33 rows (Q6_K M = 64 24.2 against 28.1 us; W4A16 M = 48..128
//    18.5-33.8 against 20.4-38.7; bf16 Q4_K M = 96 33.3 against 42.2 on
//    direct-wide); fp16 Q4_K at 49..64 only (from 96 rows direct-wide leads,
//    33.0 against 34.6 us);
//  * K = 4096 (two slices): 65..128 rows in both dtypes (W4A16 M = 96: 14.2
//    against 15.2 us fp16, 13.7 against 15.5 bf16), while the two slices'
//    tiles fit one workgroup per CU (at N = 6144 they lose, 28.3 against
//    15.8 us).
// Over at most 128 panels the split grid fills a quarter of the CUs or less
// and one panel per wave stays ahead (N = 1024, M = 96..128: 8.3-9.4
// against 12.5-14.7 us).
bool split_pays(int fmt, int dtype, long long M, long long np, long long K, int xl)
{
    const long long nch = K / kChunk, tn = (np + 3) / 4, tm = (M + 63) / 64;
    if (xl != X_FRAG || np > 256 || np <= 128 || M > 128) return false;
    if (nch >= 32 && nch < 64 && nch % 8 == 0) return M > 64 && tn * tm * 2 <= kCUs;
    if (nch < 64 || nch % 16 != 0) return false;
    if (dtype == DT_BF16 || fmt != FMT_Q4K) return M > 32;
    return M > 48 && M <= 64;
}

int mid_m_rung(int fmt, long long M, long long np, bool k2_192)
{
    const long long g64 = (M + 63) / 64, g48 = (M + 47) / 48, q = (np + 3) / 4;
    const auto rounds = [](long long wgs) { return (double)((wgs + kCUs - 1) / kCUs); };
    const double small = 8.0 * rounds(np * g64), k4 = 17.0 * rounds(q * g64);
    const double wide = fmt == FMT_Q4K ? 15.5 * rounds(q * g48) : 1e30;
    const double t192 = k2_192 ? 27.0 * rounds(((M + 191) / 192) * q) : 1e30;
    if (t192 < wide && t192 < small && t192 < k4) return RUNG_M192N64_K2;
    if (wide <= small && wide <= k4) return RUNG_WIDE;
    return small <= k4 ? RUNG_SMALL_M : RUNG_M64_K4;
}

int select_rung(int fmt, long long M, long long N, long long K, int xl, int dtype = DT_F16)
{
    const long long np = (N + 15) / 16, tn = (np + 7) / 8;
    // the direct kernels put row groups of 16 on grid.y (at most 65535);
    // beyond that only the streaming kernels' one-dimensional grid fits
    if ((M + 15) / 16 > 65535) return fmt != FMT_Q6K && stream_cost(M, np, 160) < stream_cost(M, np, 128) ? RUNG_M128N160 : RUNG_M128;
    if (np <= 4) return RUNG_SKINNY_N;
    // above 32 rows a one-panel wave carries three or four row blocks of
    // activations per weight run; four panels per wave and a grid over M win
    if (M <= 64) {
        // up to 16 rows: one panel per wave, the most waves streaming
        // weights, except over 1536 panels and more (gate and up merged),
        // where four panels per wave keep fewer, longer streams (M = 8, N =
        // 24576: Q4_K 20.2 against 23.4 us, W4A16 18.6 against 20.6), and
        // for 9..16 rows of row-major activations over 512 panels and more,
        // where each 16-row piece of X then serves four panels (M = 16, N =
        // 12288: Q4_K 12.2 against 15.7 us; on fragment-major X one panel
        // per wave wins there, 10.6 against 11.7 us)
        if (M <= 16) {
            if (np >= 1536 || (xl == X_ROW && M > 8 && np >= 512)) return RUNG_SKINNY_N;
            return RUNG_SMALL_M;
        }
        // (three row blocks per wave only pay off for Q4_K: the other
        // formats' larger raw runs spill at that size)
        if (np >= 512 && M > 16 && (M <= 32 || (M <= 48 && fmt == FMT_Q4K))) return RUNG_WIDE;
        // 49..64 rows of Q4_K (33..64 of W4A16 and Q6_K) over many panels:
        // unpack each weight once for all rows into LDS (64x64 tiles, K split
        // four ways) instead of once per 16-row group (Q6_K 12288->12288 at
        // M = 64: 50.5 against 90.1 us for direct-skinny-n)
        if (np >= 512 && ((fmt == FMT_Q4K && M > 48) || (fmt != FMT_Q4K && M > 32))) return RUNG_M64_K4;
        // Q6_K over few panels (N = 4096): 64x64 tiles with K also split
        // across workgroups, so that each CU reads a quarter of the
        // activations
        if (split_pays(fmt, dtype, M, np, K, xl)) return RUNG_M64_SK;
        // fewer panels: one panel and all rows per wave (each weight
        // unpacked once) beats four panels of 16 rows up to 64 rows
        return RUNG_SMALL_M;
    }
    const long long t128 = tn * ((M + 127) / 128), t256 = tn * ((M + 255) / 256);
    // occupancy model: a 256x128 tile counts as two 128x128 tiles; the
    // 128-row rungs as stream_cost has them (160 wide only off Q6_K)
    const double c256 = 2.0 * (double)((t256 + kCUs - 1) / kCUs);
    const double c128 = std::min(stream_cost(M, np, 128), fmt != FMT_Q6K ? stream_cost(M, np, 160) : 1e30);
    if (split_pays(fmt, dtype, M, np, K, xl)) return RUNG_M64_SK;
    if (t128 < 128) return mid_m_rung(fmt, M, np, xl == X_FRAG && (K / kChunk) % 2 == 0);
    // on fragment-major activations, a 192-row tile with K split over two
    // 6-wave groups (three waves per SIMD) whenever its tiles fit one round
    // and cover M with no more rows than 128-row tiles: 64 columns wide when
    // those tiles fit (o and down at M = 658: 36.5 and 113-119 us), else 96
    // (qkv: 47-50 us against 62 for 128x160; 192x64 would take 1.5 rounds, 64
    // us); after the 352x96 check below, the 96-wide one also over two rounds
    // at least 90% full (M = 768, N = 12288: Q4_K 90 against 101, Q6_K 254
    // against 331 us; with 1.5 or three rounds it loses to the 256-row tile)
    const long long r192 = (M + 191) / 192, t192 = r192 * ((np + 5) / 6);
    const bool even2 = xl == X_FRAG && (K / kChunk) % 2 == 0;
    const bool k2_192 = even2 && r192 * 192 <= (M + 127) / 128 * 128;
    // (the 64-wide tile pays even where it computes more padding rows: Q4_K
    // and Q6_K at M = 512, N = 4096: 29 and 85 us against 35 and 106 us for
    // the 128x128 K-split tile)
    if (even2 && r192 * ((np + 3) / 4) <= kCUs) return RUNG_M192N64_K2;
    if (k2_192 && t192 <= kCUs) return RUNG_M192N96_K2;
    // on fragment-major activations, the 352x96 tile (11 waves, three per
    // SIMD) when its rounds, each costing 1.22 rounds of the 256-row tile,
    // come out cheapest: two of its row tiles cover M = 641..704 where
    // 256-row tiles need three (merged gate_up at M = 658: 147 against 173 us;
    // M = 700, N = 12288: 76 against 95 us for 128x160; Q6_K, whose larger raw
    // runs spill four registers in it, at M = 658, N = 12288: 218 against
    // 333 us for 128x128).
    if (xl == X_FRAG) {
        const long long t352 = ((np + 5) / 6) * ((M + 351) / 352);
        const double c352 = 2.44 * (double)((t352 + kCUs - 1) / kCUs);
        if (c352 < c256 && c352 < c128) return RUNG_M352N96;
    }
    if (k2_192 && t192 <= 2 * kCUs && 10 * t192 >= 18 * kCUs) return RUNG_M192N96_K2;
    // the 256-row tile when the occupancy model has it finish no later than
    // the 128-row tiles (it unpacks each weight once for 256 rows); on
    // fragment-major activations also whenever it has 512 tiles, and for
    // Q6_K, whose unpack costs most, from one full round of them (M = 1024,
    // N = K = 12288: 363.9 against 400.4 us for 128x128)
    if (c256 <= c128 || (xl == X_FRAG && (t256 >= 512 || (fmt == FMT_Q6K && t256 >= kCUs)))) return RUNG_M16_256;
    // few tiles: split K inside the workgroup (on row-major activations only
    // over a long K, where the halves' activation reloads stay affordable)
    if (t128 <= 256 && (K >= 8192 || xl == X_FRAG)) return RUNG_M128_K2;
    // 160-wide tiles when they even out the tiles per CU (Q6_K's larger raw
    // runs do not fit that variant's registers)
    if (fmt != FMT_Q6K && stream_cost(M, np, 160) < stream_cost(M, np, 128)) return RUNG_M128N160;
    return RUNG_M128;
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
    default:
        break;
    }
    return launch_direct<FMT, DT, XL>(pl, a, s);
}

template <int XL>
hipError_t launch_xl(int fmt, int dtype, const Plan &pl, const Args &a, hipStream_t s)
{
    if (fmt == FMT_Q4K)
        return dtype == DT_F16 ? launch_fd<FMT_Q4K, DT_F16, XL>(pl, a, s) : launch_fd<FMT_Q4K, DT_BF16, XL>(pl, a, s);
    if (fmt == FMT_Q6K)
        return dtype == DT_F16 ? launch_fd<FMT_Q6K, DT_F16, XL>(pl, a, s) : launch_fd<FMT_Q6K, DT_BF16, XL>(pl, a, s);
    return dtype == DT_F16 ? launch_fd<FMT_W4, DT_F16, XL>(pl, a, s) : launch_fd<FMT_W4, DT_BF16, XL>(pl, a, s);
}

hipError_t launch(int fmt, int dtype, int xl, const Plan &pl, const Args &a, hipStream_t s)
{
    return xl == X_FRAG ? launch_xl<X_FRAG>(fmt, dtype, pl, a, s) : launch_xl<X_ROW>(fmt, dtype, pl, a, s);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A failed launch is reported once on stderr with HIP's own text; the caller
// gets QGEMM_ERR_HIP.
int launch_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return QGEMM_OK;
    fprintf(stderr, "qgemm: %s launch failed: %s (%d)\n", what, hipGetErrorString(e), (int)e);
    return QGEMM_ERR_HIP;
}

// Shape rules shared by every device entry point.
int check_shape(int fmt, long long M, long long N, long long K, long long group)
{
    if (fmt != FMT_Q4K && fmt != FMT_Q6K && fmt != FMT_W4) return QGEMM_ERR_FORMAT;
    if (M < 0 || N < 1 || K < 1) return QGEMM_ERR_SHAPE;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return QGEMM_ERR_SHAPE;
    if (fmt == FMT_W4) {  // group == 0: group size not known to the caller (rung queries)
        if (group != 0 && (group < 32 || (group & (group - 1)) != 0)) return QGEMM_ERR_FORMAT;
        if (K % 128 != 0 || (group != 0 && K % group != 0)) return QGEMM_ERR_SHAPE;
    } else if (K % 256 != 0) {
        return QGEMM_ERR_SHAPE;
    }
    return QGEMM_OK;
}

Args make_args(int fmt, const void *X, const void *W, void *Y, long long M, long long N, long long K, long long group,
               int has_zp)
{
    Args a{};
    a.X = (const uint16_t *)X;
    a.W = (const uint8_t *)W;
    a.Y = (uint16_t *)Y;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.np = (int)((N + 15) / 16);
    a.group = fmt == FMT_W4 ? (int)group : 0;
    a.has_zp = fmt == FMT_W4 ? (has_zp ? 1 : 0) : 0;
    a.kw = 1;
    if (fmt == FMT_W4) {
        a.w4_sreg = (long long)a.np * (K / 128) * 1024;
        a.w4_zreg = a.w4_sreg + (long long)a.np * (K / group) * 32;
    }
    return a;
}

// The split rung's partial sums live in a workspace kept per (device,
// stream): taken from the device's default pool in stream order the first
// time, and replaced by a larger one (the old one freed in stream order, after
// the work already queued) when a call needs more.  Workspaces are held until
// the process ends.  The lock is held across both launches of a call, so
// calls from several host threads on one stream cannot interleave them, and
// calls on different streams never share a workspace.
struct SplitWs {
    int dev;
    hipStream_t stream;
    void *p;
    size_t bytes;
};
std::mutex g_ws_mu;
std::vector<SplitWs> g_ws;

// With g_ws_mu held: a workspace of at least `bytes` for (current device, s).
// While `s` is being captured into a graph nothing is taken or returned (the
// graph would own that memory): a workspace too small then is an error, and
// one eager call on the stream beforehand provides it.
hipError_t split_workspace(hipStream_t s, size_t bytes, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(s, &cap)) != hipSuccess) return e;
    const bool capturing = cap != hipStreamCaptureStatusNone;
    bytes = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);  // whole MiB: fewer regrowths
    for (SplitWs &w : g_ws) {
        if (w.dev != dev || w.stream != s) continue;
        if (w.bytes < bytes) {
            if (capturing) return hipErrorStreamCaptureUnsupported;
            void *np = nullptr;
            if ((e = hipMallocAsync(&np, bytes, s)) != hipSuccess) return e;
            void *old = w.p;
            w.p = np;  // recorded before the old one is released, so nothing leaks if that fails
            w.bytes = bytes;
            if ((e = hipFreeAsync(old, s)) != hipSuccess) return e;
        }
        *out = w.p;
        return hipSuccess;
    }
    if (capturing) return hipErrorStreamCaptureUnsupported;
    void *np = nullptr;
    if ((e = hipMallocAsync(&np, bytes, s)) != hipSuccess) return e;
    g_ws.push_back(SplitWs{dev, s, np, bytes});
    *out = np;
    return hipSuccess;
}

int gemm_split(int fmt, int dtype, int xl, const Plan &pl, Args a, hipStream_t s)
{
    const long long MN = (long long)a.M * a.N, stride = (MN + 3) & ~3LL, rblocks = ((MN + 3) / 4 + 255) / 256;
    if (rblocks > INT32_MAX) return QGEMM_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    void *ws = nullptr;
    hipError_t e = split_workspace(s, (size_t)(stride * pl.split) * sizeof(float), &ws);
    if (e != hipSuccess) return launch_status(e, "split-K workspace");
    a.part = (float *)ws;
    a.pstride = stride;
    a.split = pl.split;
    e = launch(fmt, dtype, xl, pl, a, s);
    if (e == hipSuccess) {
        const dim3 grid((unsigned)rblocks);
        if (dtype == DT_F16)
            hipLaunchKernelGGL((k_splitk_reduce<DT_F16>), grid, dim3(256), 0, s, (const float *)ws, a.Y, MN, stride,
                               pl.split);
        else
            hipLaunchKernelGGL((k_splitk_reduce<DT_BF16>), grid, dim3(256), 0, s, (const float *)ws, a.Y, MN, stride,
                               pl.split);
        e = hipGetLastError();
    }
    return launch_status(e, kRungNames[pl.rung]);
}

int gemm(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
         long long group, int has_zp, int dtype, void *stream, int xl = X_ROW)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, M, N, K, group);
    if (st != QGEMM_OK) return st;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (rung < -1 || rung >= RUNG_COUNT) return QGEMM_ERR_FORMAT;
    if (M == 0) return QGEMM_OK;
    if (!X || !W || !Y) return QGEMM_ERR_NULL;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return QGEMM_ERR_ALIGN;
    Plan pl;
    st = make_plan(rung < 0 ? select_rung(fmt, M, N, K, xl, dtype) : rung, M, N, K, pl);
    if (st != QGEMM_OK) return st;
    Args a = make_args(fmt, X, W, Y, M, N, K, group, has_zp);
    a.kw = pl.kw;
    if (pl.rung == RUNG_M64_SK) return gemm_split(fmt, dtype, xl, pl, a, (hipStream_t)stream);
    return launch_status(launch(fmt, dtype, xl, pl, a, (hipStream_t)stream), kRungNames[pl.rung]);
}

long long packed_bytes(int fmt, long long N, long long K, long long group, int has_zp)
{
    if (fmt == FMT_Q4K) return (long long)qgemm_q4k_packed_bytes(N, K);
    if (fmt == FMT_Q6K) return (long long)qgemm_q6k_packed_bytes(N, K);
    return (long long)qgemm_w4a16_packed_bytes(N, K, group, has_zp);
}

template <int FMT, int DT>
hipError_t launch_grouped_fd(const Plan &pl, const Args &a, hipStream_t s)
{
    if (pl.rb == 1) hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 1, 4>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    else if (pl.rb == 2) hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 2, 4>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    else hipLaunchKernelGGL((k_direct_grouped<FMT, DT, 3, 4>), pl.grid, dim3(64 * pl.kw), pl.lds, s, a);
    return hipGetLastError();
}

// Grouped plan: four panels per wave, row blocks sized by the mean rows per
// expert (three 16-row blocks only for Q4_K, whose runs fit that variant),
// grid.y an upper bound on every expert's row blocks, K split as the direct
// rungs do.
// Grouped 64x64 streaming tiles (k_stream32_grouped), two waves per
// workgroup over all of K (splitting K inside the workgroup measured slower:
// too few chunks per group at an expert's K, 98-103 against 80-81 us).
template <int FMT, int DT>
hipError_t launch_grouped_stream(const Args &a, long long T, long long E, hipStream_t s)
{
    const long long tn = (a.np + 3) / 4, slots = (T + 63) / 64 + E;
    const dim3 grid((unsigned)(tn * slots));
    hipLaunchKernelGGL((k_stream32_grouped<FMT, DT, 1>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

Plan grouped_plan(int fmt, long long T, long long E, long long N, long long K)
{
    Plan pl{};
    const long long np = (N + 15) / 16, avg = (T + E - 1) / E;
    pl.rung = -1;
    pl.pn = 4;
    pl.rb = avg <= 16 ? 1 : (avg <= 32 || fmt != FMT_Q4K) ? 2 : 3;
    pl.grid = dim3((unsigned)ceil_div(np, 4), (unsigned)(ceil_div(T, 16 * pl.rb) + E), 1);
    pl.kw = pick_kw((long long)pl.grid.x * pl.grid.y, (int)(K / kChunk), false);
    pl.waves = pl.kw;
    pl.rows = 16 * pl.rb;
    pl.cols = 64;
    pl.lds = pl.kw > 1 ? (size_t)pl.kw * pl.pn * pl.rb * 64 * sizeof(float) * 4 : 0;
    return pl;
}

int grouped(int fmt, const void *X, const void *W, void *Y, const int32_t *offs, long long E, long long T, long long N,
            long long K, long long group, int has_zp, int dtype, void *stream)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, T, N, K, group);
    if (st != QGEMM_OK) return st;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (E < 1 || E > INT32_MAX / 2) return QGEMM_ERR_SHAPE;
    if (T == 0) return QGEMM_OK;
    if (!X || !W || !Y || !offs) return QGEMM_ERR_NULL;
    const long long wstride = packed_bytes(fmt, N, K, group, has_zp);
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || ((uintptr_t)offs & 3u) != 0 || wstride % 16 != 0)
        return QGEMM_ERR_ALIGN;
    if ((long long)ceil_div(T, 16) + E > 65535) return QGEMM_ERR_SHAPE;  // grid.y limit
    Args a = make_args(fmt, X, W, Y, T, N, K, group, has_zp);
    a.offs = offs;
    a.E = (int)E;
    a.wstride = wstride;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // more than 32 rows per expert on average and at least 16 chunks: 64x64
    // streaming tiles, which read an expert's activation rows once per 64
    // columns (the direct kernel reads them once per 16): 128 experts, 41
    // rows each on average, Q4_K 2048 -> 768: 80-81 against 101 us; over 6
    // chunks (Q6_K 768 -> 2048) the direct kernel stays ahead, 91 against 94
    if ((T + E - 1) / E > 32 && K / kChunk >= 16) {
        if (((N + 63) / 64) * ((T + 63) / 64 + E) > INT32_MAX) return QGEMM_ERR_SHAPE;
        if (fmt == FMT_Q4K) e = dtype == DT_F16 ? launch_grouped_stream<FMT_Q4K, DT_F16>(a, T, E, s) : launch_grouped_stream<FMT_Q4K, DT_BF16>(a, T, E, s);
        else if (fmt == FMT_Q6K) e = dtype == DT_F16 ? launch_grouped_stream<FMT_Q6K, DT_F16>(a, T, E, s) : launch_grouped_stream<FMT_Q6K, DT_BF16>(a, T, E, s);
        else e = dtype == DT_F16 ? launch_grouped_stream<FMT_W4, DT_F16>(a, T, E, s) : launch_grouped_stream<FMT_W4, DT_BF16>(a, T, E, s);
        return launch_status(e, "grouped");
    }
    const Plan pl = grouped_plan(fmt, T, E, N, K);
    a.kw = pl.kw;
    if (fmt == FMT_Q4K) e = dtype == DT_F16 ? launch_grouped_fd<FMT_Q4K, DT_F16>(pl, a, s) : launch_grouped_fd<FMT_Q4K, DT_BF16>(pl, a, s);
    else if (fmt == FMT_Q6K) e = dtype == DT_F16 ? launch_grouped_fd<FMT_Q6K, DT_F16>(pl, a, s) : launch_grouped_fd<FMT_Q6K, DT_BF16>(pl, a, s);
    else e = dtype == DT_F16 ? launch_grouped_fd<FMT_W4, DT_F16>(pl, a, s) : launch_grouped_fd<FMT_W4, DT_BF16>(pl, a, s);
    return launch_status(e, "grouped");
}

size_t staged_scratch_bytes(long long N, long long K)
{
    if (N < 1 || K < 1 || K % kChunk != 0) return 0;
    return (size_t)((N + 15) / 16) * 16 * (size_t)K * 2;
}

template <int DT>
hipError_t launch_staged_dt(int fmt, const Args &a, uint8_t *scratch, const Plan &pl, hipStream_t s)
{
    const long long work = (long long)a.np * (a.K / kChunk) * 64;
    const dim3 grid((unsigned)((work + 255) / 256));
    if (fmt == FMT_Q4K) hipLaunchKernelGGL((k_stage<FMT_Q4K, DT>), grid, dim3(256), 0, s, a, scratch);
    else if (fmt == FMT_Q6K) hipLaunchKernelGGL((k_stage<FMT_Q6K, DT>), grid, dim3(256), 0, s, a, scratch);
    else hipLaunchKernelGGL((k_stage<FMT_W4, DT>), grid, dim3(256), 0, s, a, scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.M == 0) return e;
    Args b = a;
    b.W = scratch;
    hipLaunchKernelGGL((k_stream32<FMT_DENSE, DT, 32, 8, 4, 1, 1, X_ROW>), pl.grid, dim3(256), 0, s, b);
    return hipGetLastError();
}

int staged(int fmt, const void *X, const void *W, void *scratch, size_t scratch_bytes, void *Y, long long M, long long N,
           long long K, long long group, int has_zp, int dtype, void *stream)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, M, N, K, group);
    if (st != QGEMM_OK) return st;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (!W || !scratch || (M > 0 && (!X || !Y))) return QGEMM_ERR_NULL;
    if (!aligned16(W) || !aligned16(scratch) || (M > 0 && (!aligned16(X) || !aligned16(Y)))) return QGEMM_ERR_ALIGN;
    if (scratch_bytes < staged_scratch_bytes(N, K)) return QGEMM_ERR_SIZE;
    Plan pl;
    if (int st = make_plan(RUNG_M128, M > 0 ? M : 1, N, K, pl); st != QGEMM_OK) return st;
    Args a = make_args(fmt, X, W, Y, M, N, K, group, has_zp);
    const hipError_t e = dtype == DT_F16 ? launch_staged_dt<DT_F16>(fmt, a, (uint8_t *)scratch, pl, (hipStream_t)stream)
                                         : launch_staged_dt<DT_BF16>(fmt, a, (uint8_t *)scratch, pl, (hipStream_t)stream);
    return launch_status(e, "staged");
}


// ---------------------------------------------------------------------------
// int8-activation path: rungs, validation, launches.
// ---------------------------------------------------------------------------

enum I8Rung {
    I8_M128 = 0,      // 128x128, 4 waves of 32x128
    I8_M256 = 1,      // 256x128, 8 waves of 32x128: each weight unpacked once for 256 rows
    I8_M128_K2 = 2,   // 128x128, K split over two 4-wave groups
    I8_M256N96 = 3,   // 256x96, 8 waves of 32x96
    I8_M512N96 = 4,   // 512x96, 8 waves of 64x96: each weight unpacked once for 512 rows
    I8_M352N96 = 5,   // 352x96, 11 waves of 32x96 (three per SIMD)
    I8_M192N96_K2 = 6,  // 192x96, K split over two 6-wave groups (three waves per SIMD)
    I8_M192N64_K2 = 7,  // 192x64, K split over two 6-wave groups
    I8_M64_SK = 8,      // 64x64, K split over four groups and across workgroups
    I8_RUNG_COUNT = 9
};
const char *const kI8RungNames[I8_RUNG_COUNT] = {"i8-128x128",   "i8-256x128",   "i8-128x128-k2",
                                                   "i8-256x96",    "i8-512x96",    "i8-352x96",
                                                   "i8-192x96-k2", "i8-192x64-k2", "i8-64x64-sk"};
// int32 sums stay exact while K * 127 * 127 < 2^31
constexpr long long kI8MaxK = 131072;

int i8_plan(int rung, long long M, long long N, long long K, Plan &pl)
{
    pl = Plan{};
    pl.rung = rung;
    pl.kw = 1;
    pl.split = 1;
    const int nch = (int)(K / kChunk);
    switch (rung) {
    case I8_M128: pl.rows = 128; pl.cols = 128; pl.waves = 4; break;
    case I8_M256: pl.rows = 256; pl.cols = 128; pl.waves = 8; break;
    case I8_M128_K2:
        pl.rows = 128;
        pl.cols = 128;
        pl.kw = (K / kChunk) % 2 == 0 ? 2 : 1;
        pl.waves = 4 * pl.kw;
        break;
    case I8_M256N96: pl.rows = 256; pl.cols = 96; pl.waves = 8; break;
    case I8_M512N96: pl.rows = 512; pl.cols = 96; pl.waves = 8; break;
    case I8_M352N96: pl.rows = 352; pl.cols = 96; pl.waves = 11; break;
    case I8_M192N96_K2:
    case I8_M192N64_K2:
        pl.rows = 192;
        pl.cols = rung == I8_M192N64_K2 ? 64 : 96;
        pl.kw = (K / kChunk) % 2 == 0 ? 2 : 1;
        pl.waves = 6 * pl.kw;
        break;
    case I8_M64_SK:
        pl.rows = 64;
        pl.cols = 64;
        pl.kw = nch % 4 == 0 ? 4 : nch % 2 == 0 ? 2 : 1;
        pl.waves = 2 * pl.kw;
        break;
    default: return QGEMM_ERR_FORMAT;
    }
    const long long np = (N + 15) / 16;
    const long long tn = (np + pl.cols / 16 - 1) / (pl.cols / 16), tm = (M + pl.rows - 1) / pl.rows;
    if (tn * tm > INT32_MAX) return QGEMM_ERR_SHAPE;
    pl.tiles_n = (int)tn;
    pl.tiles_m = (int)tm;
    if (rung == I8_M64_SK) {
        // slices across workgroups: double while the grid stays within two
        // workgroups per CU, the slices divide the chunks evenly among the
        // in-group K groups and each group keeps two chunks
        while (pl.split < 8 && tn * tm * 2 * pl.split <= 2 * kCUs && nch % (2 * pl.split * pl.kw) == 0 &&
               nch / (2 * pl.split * pl.kw) >= 2)
            pl.split *= 2;
    }
    if (tn * tm * pl.split > INT32_MAX) return QGEMM_ERR_SHAPE;
    pl.grid = dim3((unsigned)(tn * tm * pl.split), 1, 1);
    return QGEMM_OK;
}

// The int8 ladder (measured on MI355X, Q4_K/Q6_K/W4A16, M = 16..4096).
// The unpack costs about four VALU instructions per weight, so a tile is
// VALU-bound unless many rows share each unpacked weight:
//  * with an even chunk count, a 192-row tile with K split over two 6-wave
//    groups (three waves per SIMD) when its tiles fit one round, even where
//    it computes more padding rows: 64 columns wide when those tiles fit (o
//    and down at M = 658: 25.0 and 64.0 us against 28.7 and 75.5 us for
//    192x96), else 96 (qkv: 32.1 us against 34.5 on 256x96 and 43 on
//    192x64; Q6_K M = 512, N = 4096: 72 against 84 us for the 128x128
//    K-split tile);
//  * at most 256 tiles of 128x128 (and an even chunk count): the 128x128
//    tile with K split over two wave groups (o and down at M = 658);
//  * up to 128 rows: the 128x128 tile;
//  * otherwise the 256x128, 256x96, 352x96 or 512x96 tile, whichever
//    finishes in the fewest rounds of one workgroup per CU, a round costing
//    1, 0.85, 1.17 and 1.35 (fitted to the measured times: the merged
//    gate_up at M = 658 91 us on 352x96 against 107 on 256x96 and 117 on
//    256x128; M = 2048 121 us on 512x96 against 133 on 256x128 and 138 on
//    352x96; M = 4096 238 against 260 and 268).  The 352-row tile runs three
//    waves per SIMD and unpacks each weight for 352 rows: two of its row
//    tiles cover M = 658 where 256-row tiles need three.
int i8_select(int fmt, long long M, long long N, long long K)
{
    const long long np = (N + 15) / 16, t128 = ((M + 127) / 128) * ((np + 7) / 8), r192 = (M + 191) / 192;
    const long long nch = K / kChunk;
    // few tiles of 192x64 (at most half the CUs): 64x64 tiles with K split
    // across workgroups as well, up to 64 rows (Q6_K, whose unpack weighs
    // most, up to 256): Q6_K 12288->4096 at M = 16..256 28.6-56.1 against
    // 59.4-64.3 us, Q4_K 4096->4096 at M = 16..64 15.2-17.0 against
    // 23.5-24.1 us (row quantizer included); over more tiles, or Q4_K from
    // 96 rows, the 192x64 tile wins (4096->12288: 23.7-25.7 against 24.2-26.3)
    if (nch % 8 == 0 && nch >= 16 && r192 * ((np + 3) / 4) <= kCUs / 2 && (M <= 64 || (fmt == FMT_Q6K && M <= 256)))
        return I8_M64_SK;
    if ((K / kChunk) % 2 == 0 && r192 * ((np + 3) / 4) <= kCUs) return I8_M192N64_K2;
    if ((K / kChunk) % 2 == 0 && r192 * ((np + 5) / 6) <= kCUs) return I8_M192N96_K2;
    if (t128 <= 256 && (K / kChunk) % 2 == 0) return I8_M128_K2;
    if (M <= 128) return I8_M128;
    const long long tm256 = (M + 255) / 256, tm352 = (M + 351) / 352, tm512 = (M + 511) / 512;
    const long long tn128 = (np + 7) / 8, tn96 = (np + 5) / 6;
    const auto rounds = [](long long tiles) { return (double)((tiles + kCUs - 1) / kCUs); };
    const double c[4] = {rounds(tm256 * tn128), 0.85 * rounds(tm256 * tn96), 1.17 * rounds(tm352 * tn96),
                         1.35 * rounds(tm512 * tn96)};
    const int rung[4] = {I8_M256, I8_M256N96, I8_M352N96, I8_M512N96};
    int best = 0;
    for (int i = 1; i < 4; i++)
        if (c[i] < c[best]) best = i;
    return rung[best];
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
    const bool slower2 = (FMT == FMT_W4 && pl.rung == I8_M256N96) || pl.rung == I8_M192N96_K2 ||
                         (FMT == FMT_Q6K && (pl.rung == I8_M512N96 || pl.rung == I8_M352N96));
    if (!slower2 && (a.K / kChunk) % (2 * pl.kw) == 0) return launch_i8_cpb<FMT, DT, 2>(pl.rung, pl, a, s);
    return launch_i8_cpb<FMT, DT, 1>(pl.rung, pl, a, s);
}

template <int DT>
hipError_t launch_i8_dt(int fmt, const Plan &pl, const Args &a, hipStream_t s)
{
    if (fmt == FMT_Q4K) return launch_i8_fd<FMT_Q4K, DT>(pl, a, s);
    if (fmt == FMT_Q6K) return launch_i8_fd<FMT_Q6K, DT>(pl, a, s);
    return launch_i8_fd<FMT_W4, DT>(pl, a, s);
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int i8_gemm(int fmt, int rung, const void *Xq, const float *sx, const void *W, const float *rw, const float *sw,
            void *Y, long long M, long long N, long long K, long long group, int has_zp, int dtype, void *stream)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, M, N, K, group);
    if (st != QGEMM_OK) return st;
    if (K > kI8MaxK) return QGEMM_ERR_SHAPE;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (rung < -1 || rung >= I8_RUNG_COUNT) return QGEMM_ERR_FORMAT;
    if (M == 0) return QGEMM_OK;
    if (!Xq || !sx || !W || !rw || !sw || !Y) return QGEMM_ERR_NULL;
    if (!aligned16(Xq) || !aligned16(W) || !aligned16(Y) || !aligned4(sx) || !aligned4(rw) || !aligned4(sw))
        return QGEMM_ERR_ALIGN;
    Plan pl;
    st = i8_plan(rung < 0 ? i8_select(fmt, M, N, K) : rung, M, N, K, pl);
    if (st != QGEMM_OK) return st;
    Args a = make_args(fmt, Xq, W, Y, M, N, K, group, has_zp);
    a.sx = sx;
    a.rw = rw;
    a.sw = sw;
    if (pl.rung == I8_M64_SK) {
        // int32 partial sums per K slice in the per-stream workspace, then
        // their exact total through the unsplit epilogue
        const hipStream_t s = (hipStream_t)stream;
        const long long MN = M * N, stride = (MN + 3) & ~3LL, rblocks = ((MN + 3) / 4 + 255) / 256;
        if (rblocks > INT32_MAX) return QGEMM_ERR_SHAPE;
        std::lock_guard<std::mutex> lock(g_ws_mu);
        void *ws = nullptr;
        hipError_t e = split_workspace(s, (size_t)(stride * pl.split) * sizeof(int), &ws);
        if (e != hipSuccess) return launch_status(e, "split-K workspace");
        a.part = (float *)ws;
        a.pstride = stride;
        a.split = pl.split;
        e = dtype == DT_F16 ? launch_i8_dt<DT_F16>(fmt, pl, a, s) : launch_i8_dt<DT_BF16>(fmt, pl, a, s);
        if (e == hipSuccess) {
            if (dtype == DT_F16)
                hipLaunchKernelGGL((k_i8_splitk_reduce<DT_F16>), dim3((unsigned)rblocks), dim3(256), 0, s,
                                   (const int *)ws, sx, sw, (uint16_t *)Y, (int)M, (int)N, stride, pl.split);
            else
                hipLaunchKernelGGL((k_i8_splitk_reduce<DT_BF16>), dim3((unsigned)rblocks), dim3(256), 0, s,
                                   (const int *)ws, sx, sw, (uint16_t *)Y, (int)M, (int)N, stride, pl.split);
            e = hipGetLastError();
        }
        return launch_status(e, kI8RungNames[pl.rung]);
    }
    const hipError_t e = dtype == DT_F16 ? launch_i8_dt<DT_F16>(fmt, pl, a, (hipStream_t)stream)
                                         : launch_i8_dt<DT_BF16>(fmt, pl, a, (hipStream_t)stream);
    return launch_status(e, kI8RungNames[pl.rung]);
}

int i8_quantize(const void *X, void *Xq, float *sx, long long M, long long K, int dtype, void *stream)
{
    // one wave per padded row: the grid fits while M + 31 does
    if (M < 0 || K < 32 || K % 32 != 0 || M > INT32_MAX - 31 || K > INT32_MAX) return QGEMM_ERR_SHAPE;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (M == 0) return QGEMM_OK;
    if (!X || !Xq || !sx) return QGEMM_ERR_NULL;
    if (!aligned16(X) || !aligned16(Xq) || !aligned4(sx)) return QGEMM_ERR_ALIGN;
    const unsigned groups = (unsigned)((M + 31) / 32 * 8);  // four padded rows per workgroup
    hipStream_t s = (hipStream_t)stream;
    if (dtype == DT_F16)
        hipLaunchKernelGGL((k_i8_quant<DT_F16>), dim3(groups), dim3(256), 0, s, (const uint16_t *)X, (uint8_t *)Xq, sx,
                           (int)M, (int)K);
    else
        hipLaunchKernelGGL((k_i8_quant<DT_BF16>), dim3(groups), dim3(256), 0, s, (const uint16_t *)X, (uint8_t *)Xq, sx,
                           (int)M, (int)K);
    return launch_status(hipGetLastError(), "i8 quantize");
}

int i8_colscale(int fmt, const void *W, float *rw, float *sw, long long N, long long K, long long group, int has_zp,
                void *stream)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, 0, N, K, group);
    if (st != QGEMM_OK) return st;
    if (!W || !rw || !sw) return QGEMM_ERR_NULL;
    if (!aligned16(W) || !aligned4(rw) || !aligned4(sw)) return QGEMM_ERR_ALIGN;
    Args a = make_args(fmt, nullptr, W, nullptr, 0, N, K, group, has_zp);
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)a.np);
    if (fmt == FMT_Q4K) hipLaunchKernelGGL((k_i8_colscale<FMT_Q4K>), grid, dim3(64), 0, s, a, rw, sw);
    else if (fmt == FMT_Q6K) hipLaunchKernelGGL((k_i8_colscale<FMT_Q6K>), grid, dim3(64), 0, s, a, rw, sw);
    else hipLaunchKernelGGL((k_i8_colscale<FMT_W4>), grid, dim3(64), 0, s, a, rw, sw);
    return launch_status(hipGetLastError(), "i8 colscale");
}

void fill_info(const Plan &pl, int32_t *info)
{
    info[0] = pl.rung;
    info[1] = pl.rows;
    info[2] = pl.cols;
    info[3] = kChunk;
    info[4] = pl.waves;
    info[5] = pl.kw * std::max(pl.split, 1);
    info[6] = pl.tiles_n;
    info[7] = pl.tiles_m;
}

}  // namespace

extern "C" {

const char *qgemm_status_str(int status)
{
    switch (status) {
    case QGEMM_OK: return "ok";
    case QGEMM_ERR_NULL: return "null pointer";
    case QGEMM_ERR_SHAPE: return "illegal shape";
    case QGEMM_ERR_DTYPE: return "unsupported dtype";
    case QGEMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QGEMM_ERR_FORMAT: return "unsupported format, group size or rung";
    case QGEMM_ERR_SIZE: return "buffer too small";
    case QGEMM_ERR_HIP: return "HIP launch failed";
    case QGEMM_ERR_INPUT: return "malformed input data";
    default: return "unknown status";
    }
}

int qgemm_q4k(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int dtype, void *stream)
{
    return gemm(FMT_Q4K, -1, X, W, Y, M, N, K, 0, 0, dtype, stream);
}

int qgemm_q6k(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int dtype, void *stream)
{
    return gemm(FMT_Q6K, -1, X, W, Y, M, N, K, 0, 0, dtype, stream);
}

int qgemm_w4a16(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int64_t group_size,
                int has_zp, int dtype, void *stream)
{
    return gemm(FMT_W4, -1, X, W, Y, M, N, K, group_size, has_zp, dtype, stream);
}

int qgemm_gemm_rung(int format, int rung, const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K,
                    int64_t group_size, int has_zp, int dtype, void *stream)
{
    return gemm(format, rung, X, W, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, stream);
}

int qgemm_num_rungs(void) { return RUNG_COUNT; }

const char *qgemm_rung_name(int rung) { return rung >= 0 && rung < RUNG_COUNT ? kRungNames[rung] : nullptr; }

int qgemm_rung_info(int rung, int format, int64_t M, int64_t N, int64_t K, int dtype, int32_t *info8)
{
    if (!info8) return QGEMM_ERR_NULL;
    int st = check_shape(format, M, N, K, 0);
    if (st != QGEMM_OK) return st;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    Plan pl;
    st = make_plan(rung, M, N, K, pl);
    if (st != QGEMM_OK) return st;
    fill_info(pl, info8);
    return QGEMM_OK;
}

int qgemm_select_rung(int format, int64_t M, int64_t N, int64_t K, int dtype, int32_t *info8)
{
    return qgemm_rung_info(select_rung(format, M, N, K, X_ROW, dtype), format, M, N, K, dtype, info8);
}

int qgemm_select_rung_xf(int format, int64_t M, int64_t N, int64_t K, int dtype, int32_t *info8)
{
    return qgemm_rung_info(select_rung(format, M, N, K, X_FRAG, dtype), format, M, N, K, dtype, info8);
}

size_t qgemm_xf_bytes(int64_t M, int64_t K)
{
    if (M < 0 || K < kChunk || K % kChunk != 0 || M > INT32_MAX || K > INT32_MAX) return 0;
    return (size_t)((M + 31) / 32) * 32 * (size_t)K * 2;
}

int qgemm_x_to_xf(const void *X, void *Xf, int64_t M, int64_t K, void *stream)
{
    if (M < 0 || K < kChunk || K % kChunk != 0 || M > INT32_MAX || K > INT32_MAX) return QGEMM_ERR_SHAPE;
    const long long tiles = ((M + 31) / 32) * (K / kChunk);
    if (tiles > INT32_MAX) return QGEMM_ERR_SHAPE;
    if (M == 0) return QGEMM_OK;
    if (!X || !Xf) return QGEMM_ERR_NULL;
    if (!aligned16(X) || !aligned16(Xf)) return QGEMM_ERR_ALIGN;
    hipLaunchKernelGGL(k_x_to_xf, dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)stream, (const uint16_t *)X,
                       (uint16_t *)Xf, (int)M, (int)K);
    return launch_status(hipGetLastError(), "x_to_xf");
}

int qgemm_gemm_xf(int format, int rung, const void *Xf, const void *W, void *Y, int64_t M, int64_t N, int64_t K,
                  int64_t group_size, int has_zp, int dtype, void *stream)
{
    return gemm(format, rung, Xf, W, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, stream, X_FRAG);
}

int qgemm_dequant(int format, const void *W, void *Wout, int64_t N, int64_t K, int64_t group_size, int has_zp,
                  int dtype, void *stream)
{
    if (format == FMT_W4 && group_size == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(format, 0, N, K, format == FMT_W4 ? group_size : 0);
    if (st != QGEMM_OK) return st;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (!W || !Wout) return QGEMM_ERR_NULL;
    if (!aligned16(W) || !aligned16(Wout)) return QGEMM_ERR_ALIGN;
    Args a = make_args(format, nullptr, W, nullptr, 0, N, K, group_size, has_zp);
    const long long total = (long long)a.np * (K / kChunk) * 64;
    dim3 grid((unsigned)((total + 255) / 256));
    hipStream_t s = (hipStream_t)stream;
    uint16_t *o = (uint16_t *)Wout;
#define QG_DQ(F, D) hipLaunchKernelGGL((k_dequant<F, D>), grid, dim3(256), 0, s, a, o)
    if (format == FMT_Q4K) { if (dtype == DT_F16) QG_DQ(FMT_Q4K, DT_F16); else QG_DQ(FMT_Q4K, DT_BF16); }
    else if (format == FMT_Q6K) { if (dtype == DT_F16) QG_DQ(FMT_Q6K, DT_F16); else QG_DQ(FMT_Q6K, DT_BF16); }
    else { if (dtype == DT_F16) QG_DQ(FMT_W4, DT_F16); else QG_DQ(FMT_W4, DT_BF16); }
#undef QG_DQ
    return launch_status(hipGetLastError(), "dequant");
}

size_t qgemm_staged_scratch_bytes(int64_t N, int64_t K)
{
    return staged_scratch_bytes(N, K);
}

int qgemm_staged(int format, const void *X, const void *Wpacked, void *scratch, size_t scratch_bytes, void *Y, int64_t M,
                 int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream)
{
    return staged(format, X, Wpacked, scratch, scratch_bytes, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype,
                  stream);
}

int qgemm_grouped(int format, const void *X, const void *Wpacked, void *Y, const int32_t *offsets, int64_t E, int64_t T,
                  int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream)
{
    return grouped(format, X, Wpacked, Y, offsets, E, T, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, stream);
}

size_t qgemm_i8_xq_bytes(int64_t M, int64_t K)
{
    if (M < 0 || K < 32 || K % 32 != 0 || M > INT32_MAX - 31 || K > INT32_MAX) return 0;
    return (size_t)((M + 31) / 32) * 32 * (size_t)K;
}

int qgemm_i8_quantize(const void *X, void *Xq, float *sx, int64_t M, int64_t K, int dtype, void *stream)
{
    return i8_quantize(X, Xq, sx, M, K, dtype, stream);
}

int qgemm_i8_colscale(int format, const void *Wpacked, float *rw, float *sw, int64_t N, int64_t K, int64_t group_size,
                      int has_zp, void *stream)
{
    return i8_colscale(format, Wpacked, rw, sw, N, K, format == FMT_W4 ? group_size : 0, has_zp, stream);
}

int qgemm_i8_gemm(int format, int rung, const void *Xq, const float *sx, const void *Wpacked, const float *rw,
                  const float *sw, void *Y, int64_t M, int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype,
                  void *stream)
{
    return i8_gemm(format, rung, Xq, sx, Wpacked, rw, sw, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype,
                   stream);
}

int qgemm_i8_num_rungs(void) { return I8_RUNG_COUNT; }

const char *qgemm_i8_rung_name(int rung) { return rung >= 0 && rung < I8_RUNG_COUNT ? kI8RungNames[rung] : nullptr; }

int qgemm_i8_rung_info(int rung, int format, int64_t M, int64_t N, int64_t K, int32_t *info8)
{
    if (!info8) return QGEMM_ERR_NULL;
    int st = check_shape(format, M, N, K, 0);
    if (st != QGEMM_OK) return st;
    if (K > kI8MaxK) return QGEMM_ERR_SHAPE;
    Plan pl;
    st = i8_plan(rung, M, N, K, pl);
    if (st != QGEMM_OK) return st;
    fill_info(pl, info8);
    return QGEMM_OK;
}

int qgemm_i8_select_rung(int format, int64_t M, int64_t N, int64_t K, int32_t *info8)
{
    return qgemm_i8_rung_info(i8_select(format, M, N, K), format, M, N, K, info8);
}

}  // extern "C"
