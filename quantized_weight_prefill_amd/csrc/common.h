// common.h -- what every kernel of the fused-dequant prefill GEMM shares
// (gfx950, CDNA4): launch arguments, activation layouts, the tile order, the
// weight-run loads and the unpack, the MFMA wrappers and the epilogue stores.
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
//   * one mixed-precision FMA per weight (fp16 input, binary32 arithmetic)
//     forms factor*q - bias as the batched-prefill post's shader does ("The
//     fix: K-parallel batched DMMV"), with factor scaled by 2^24 to cancel
//     the code's scale, and the result is converted to the operand type.
//
// Every product d*sc, dmin*m, d*s, s*zp is exact in binary32.  fp16 weights
// come from v_fma_mix, which rounds the exact code*factor - bias once into
// fp16.  bf16 weights go through a binary32 FMA result and one conversion:
// exact whenever the exact weight fits binary32 (always for Q6_K and W4A16,
// and for Q4_K whenever the exponents of d and dmin differ by at most 3);
// other bf16 Q4_K runs take exact_round (a two-sum and rounding to odd).
//
// MFMA operands are used "transposed": the weight fragment is the A operand
// and the activation fragment the B operand, so the accumulator holds Y^T and
// each lane ends with four consecutive output columns of one row (one 8-byte
// store).  The K order inside one MFMA is a free permutation as long as both
// operands agree; each kernel picks the one that lets a lane's 32-code run
// fill whole fragments.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "qgemm.h"

namespace qg {

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
// the operand pair w_lo, w_hi with w = code*2^-24 * fa + nb rounded into the
// operand type.
template <int DT>
__device__ __forceinline__ uint32_t dq_pair(uint32_t t, float fa, float nb);

// fp16: the FMA and the conversion compile to one v_fma_mix{lo,hi}_f16 per
// weight, which widens the fp16 code exactly, forms code*fa + nb without an
// intermediate rounding and rounds that once into fp16 -- the single
// rounding of the exact value that the unpack contract asks for, for every
// Q4_K d/dmin pair as well.  (A binary32 FMA followed by a conversion would
// round twice; the test suite checks the compiled kernels for that form.)
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

// Weight of an exact value qs*fa + nb whose binary32 sum may be inexact (Q4_K
// with d and dmin far apart), rounded once into fp16 or bf16.  qs*fa and nb
// are exact binary32 values; a two-sum (Knuth) gives the error of their
// binary32 sum, which is then replaced by the sum rounded to odd (truncated
// toward zero, last bit set when inexact).  Rounding that value to nearest
// even in a format with at least two significand bits fewer than binary32
// gives the rounding of the exact value (Boldo and Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// 2008); fp16 (11 bits, its subnormal grid included) and bf16 (8) qualify.
template <int DT>
__device__ __forceinline__ uint16_t exact_round(float qs, float fa, float nb)
{
#pragma clang fp contract(off)
    const float A = qs * fa;  // exact: at most 21 significant bits
    const float s = A + nb;
    const float bb = s - A;
    const float e = (A - (s - bb)) + (nb - bb);
    uint32_t sb = __builtin_bit_cast(uint32_t, s);
    if (e != 0.0f) {
        // s is nonzero here (a binary32 sum that rounds to zero is exact)
        if ((e > 0.0f) != (s > 0.0f)) sb -= 1u;  // one step toward zero: the truncation
        sb |= 1u;
    }
    const float o = __builtin_bit_cast(float, sb);
    if constexpr (DT == DT_F16) return __builtin_bit_cast(uint16_t, (_Float16)o);
    else return __builtin_bit_cast(uint16_t, (__bf16)o);
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
    bool exact;      // bf16 Q4_K run whose values may not fit binary32 (d, dmin far apart)
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
            // bf16 goes through a binary32 FMA result: exact (so the
            // conversion is the one rounding) whenever the exponent fields
            // of d and dmin differ by at most 3 (a subnormal counts as
            // exponent 1); other runs take exact_round
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
template <int DT>
__device__ __noinline__ u32x4 unpack_word_exact(u32x4 codes, float fa, float nb, int i)
{
    u32x4 out;
    const uint32_t x = codes[i], x8 = x >> 8;
    const uint32_t t[4] = {x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u};
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const f16x2 h = __builtin_bit_cast(f16x2, t[p]);
        const float f = (p & 1) ? fa * 0.0625f : fa;
        out[p] = (uint32_t)exact_round<DT>((float)h.x, f, nb) | ((uint32_t)exact_round<DT>((float)h.y, f, nb) << 16);
    }
    return out;
}

template <int FMT, int DT>
__device__ __forceinline__ u32x4 unpack_word_any(const RunRaw<FMT> &u, const RunParams &pr, int i)
{
    if constexpr (FMT == FMT_Q4K && DT == DT_BF16) {
        if (pr.exact) return unpack_word_exact<DT>(u.codes, pr.fa, pr.nb, i);
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

// 32x32x16 MFMA: twice the MACs of the 16x16x32 form per instruction, each
// operand fragment feeding 32 rows or columns instead of 16.
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

}  // namespace qg
