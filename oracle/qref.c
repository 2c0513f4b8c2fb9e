/*
 * qref.c -- plain, slow CPU oracle for the quantized-weight prefill linear
 * layer  Y[M,N] = X[M,K] . dequant(W)[K,N].
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library, and it never calls it.
 *
 * What it computes (each step cites the passage it follows):
 *
 *  1. Field decode of the stored weight formats, scalar and byte by byte:
 *     Q4_K (fp16 d and dmin, eight 6-bit sub-block scales and mins, 4-bit
 *     codes; 144 bytes per 256 weights -- the dequant-scratch post, "The two
 *     passes hiding inside one matmul"), Q6_K (6-bit codes split into a low
 *     nibble and a high 2-bit pair, one int8 scale per 16 weights, fp16 d;
 *     210 bytes per 256 weights) and W4A16 (4-bit codes, an fp16 scale and a
 *     4-bit zero-point per group of K -- the vLLM W4A16 PR, section 1
 *     "Packed fp16 dequant").  The byte order inside the k-quant blocks is
 *     the GGUF convention, which the pages do not spell out.
 *
 *  2. The unpacked weight, in the activation type t (fp16 or bf16):
 *        Q4_K : w = RN_t( d*sc*q - dmin*m )     (factor*q - bias, factor = d*sc, bias = dmin*m)
 *        Q6_K : w = RN_t( d*s*(q - 32) )
 *        W4A16: w = RN_t( s*(q - zp) )
 *     RN_t is ONE round-to-nearest-even of the exact value into t: the W4A16
 *     PR (section 1) subtracts exactly and lets the multiply that follows
 *     round once; the same single rounding is read for the k-quants, whose
 *     weight is the batched-prefill post's factor*q - bias ("The fix:
 *     K-parallel batched DMMV").  Every rounding below is done on exact
 *     integers (value = n * 2^e), so nothing depends on the host's FPU.
 *
 *  3. Yref[m][n] = sum_k X[m][k] * W[k][n] in fp64, a naive triple loop
 *     (the k loop innermost, W read through a transposed copy), together with
 *     the error scale B[m][n] = sum_k |X[m][k]| * |W[k][n]|.
 *
 *  4. The fragment-major copy of X, an activation layout of the library
 *     under test (not of the pages): element (m, k) of X [M][K] moves to
 *        ((m/32 * K/128 + k/128) * 8 + (k/16)%8) * 512 + ((k/8)%2 * 32 + m%32) * 8 + k%8
 *     and rows M .. 32*ceil(M/32)-1 are zero.  It only moves bit patterns.
 *
 *  5. The int8-activation variant (the batched-prefill PR's single-pass row
 *     quantize feeding an int8-native GEMM, and the prefill post's closing
 *     remark that activation quantization and weight dequant fusion are one
 *     idea applied to the two operands).  The pages fix neither the scale
 *     granularity nor the rounding; the reading implemented here:
 *       - weights: w32 = RN_f32(exact step-2 value); per output column n,
 *         amax_n = max_k |w32|, r_n = RN_f32(127/amax_n), s_n = RN_f32(amax_n/127)
 *         (both 0 when amax_n < 2^-96, a bound that only a bf16 row can go
 *         below, where 127/amax would leave binary32); qw = RNE_int(w32 * r_n),
 *         the product exact;
 *       - activations: per row m the same with x (exact in binary32):
 *         r_m = RN_f32(127/amax_m), s_m = RN_f32(amax_m/127), qx = RNE_int(x * r_m);
 *       - Y[m][n] = RN_t( RN_f32( RN_f32(acc) * RN_f32(s_m * s_n) ) ),
 *         acc = sum_k qx * qw exactly (an integer).
 *     127/amax and amax/127 are formed in binary64 and rounded once more to
 *     binary32; that second rounding is innocuous for a quotient since
 *     53 >= 2*24 + 2 (Figueroa, "When is double rounding innocuous?", 1995),
 *     so both equal the exact quotient rounded once.  The int8 activation
 *     copy also has a fragment-major layout of the library under test:
 *        Q[m][k] at (m/32)*32*K + (k/32)*1024 + (k/16)%2*512 + (m%32)*16 + k%16,
 *     rows M .. 32*ceil(M/32)-1 zero.
 *
 * All 16-bit floating-point values cross this interface as raw bit patterns
 * (uint16_t).  dtype 0 = fp16, 1 = bf16.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define QREF_F16 0
#define QREF_BF16 1

/* ------------------------------------------------------------------------ */
/* Exact rounding of n * 2^e into a binary format                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t n; /* signed integer significand */
    int e;     /* value = n * 2^e */
    int inf;   /* +-1 when the rounded value overflowed */
    int neg;   /* sign, kept when a nonzero value rounds to zero */
} xval;

static int bitlen(uint64_t a) { return a ? 64 - __builtin_clzll(a) : 0; }

/* Round n*2^e to the nearest value with p significand bits, normal exponent
 * range [emin, emax], ties to even; values below 2^emin round on the fixed
 * subnormal grid 2^(emin-p+1).  Requires |n| < 2^62. */
static xval round_exact(int64_t n, int e, int p, int emin, int emax)
{
    xval r = {0, 0, 0, n < 0};
    if (n == 0) return r;
    int neg = n < 0;
    uint64_t a = neg ? (uint64_t)(-n) : (uint64_t)n;
    int E = bitlen(a) - 1 + e;                      /* a*2^e in [2^E, 2^(E+1)) */
    int qexp = (E < emin ? emin : E) - (p - 1);     /* exponent of one ulp      */
    int shift = qexp - e;
    uint64_t q;
    if (shift <= 0) {
        q = a;
        qexp = e;
    } else if (shift >= 63) {
        q = 0; /* a < 2^62 <= half an ulp */
    } else {
        q = a >> shift;
        uint64_t rem = a & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (q & 1))) q++;
    }
    if (q == 0) return r;
    if (bitlen(q) - 1 + qexp > emax) {
        r.inf = neg ? -1 : 1;
        return r;
    }
    r.n = neg ? -(int64_t)q : (int64_t)q;
    r.e = qexp;
    return r;
}

static xval rn_f32(int64_t n, int e) { return round_exact(n, e, 24, -126, 127); }
static xval rn_f16(int64_t n, int e) { return round_exact(n, e, 11, -14, 15); }
static xval rn_bf16(int64_t n, int e) { return round_exact(n, e, 8, -126, 127); }

/* Bit pattern of an exactly representable rounded value. */
static uint16_t enc_f16(xval v)
{
    if (v.inf) return v.inf < 0 ? 0xFC00 : 0x7C00;
    if (v.n == 0) return v.neg ? 0x8000 : 0;
    uint16_t s = v.n < 0 ? 0x8000 : 0;
    uint64_t a = v.n < 0 ? (uint64_t)(-v.n) : (uint64_t)v.n;
    int E = bitlen(a) - 1 + v.e;
    if (E < -14) { /* subnormal: a*2^e = mant*2^-24 */
        return s | (uint16_t)(a << (v.e + 24));
    }
    int sh = v.e - (E - 10); /* bring significand to 11 bits */
    uint64_t sig = sh >= 0 ? a << sh : a >> (-sh);
    return s | (uint16_t)((E + 15) << 10) | (uint16_t)(sig - 1024);
}

static uint16_t enc_bf16(xval v)
{
    if (v.inf) return v.inf < 0 ? 0xFF80 : 0x7F80;
    if (v.n == 0) return v.neg ? 0x8000 : 0;
    uint16_t s = v.n < 0 ? 0x8000 : 0;
    uint64_t a = v.n < 0 ? (uint64_t)(-v.n) : (uint64_t)v.n;
    int E = bitlen(a) - 1 + v.e;
    if (E < -126) {
        return s | (uint16_t)(a << (v.e + 133));
    }
    int sh = v.e - (E - 7);
    uint64_t sig = sh >= 0 ? a << sh : a >> (-sh);
    return s | (uint16_t)((E + 127) << 7) | (uint16_t)(sig - 128);
}

/* fp16 bits -> (integer significand, exponent); returns -1 for inf/nan. */
static int f16_split(uint16_t h, int64_t *n, int *e)
{
    int ex = (h >> 10) & 31, mant = h & 1023;
    if (ex == 31) return -1;
    int64_t sig = ex ? (1024 + mant) : mant;
    *e = ex ? ex - 25 : -24;
    *n = (h & 0x8000) ? -sig : sig;
    return 0;
}

double qref_f16_to_double(uint16_t h)
{
    int ex = (h >> 10) & 31, mant = h & 1023;
    double s = (h & 0x8000) ? -1.0 : 1.0;
    if (ex == 31) return mant ? NAN : s * INFINITY;
    if (ex == 0) return s * ldexp((double)mant, -24);
    return s * ldexp((double)(1024 + mant), ex - 25);
}

double qref_bf16_to_double(uint16_t b)
{
    int ex = (b >> 7) & 255, mant = b & 127;
    double s = (b & 0x8000) ? -1.0 : 1.0;
    if (ex == 255) return mant ? NAN : s * INFINITY;
    if (ex == 0) return s * ldexp((double)mant, -133);
    return s * ldexp((double)(128 + mant), ex - 134);
}

static double t_to_double(uint16_t v, int dtype)
{
    return dtype == QREF_F16 ? qref_f16_to_double(v) : qref_bf16_to_double(v);
}

/* Round-to-nearest-even of a finite double into fp16 / bf16 / binary32 bits.
 * Exposed so the tests can pin the rounding against library conversions. */
static int double_split(double x, int64_t *n, int *e)
{
    if (!isfinite(x)) return -1;
    if (x == 0.0) { *n = 0; *e = 0; return 0; }
    int ex;
    double fr = frexp(x, &ex);              /* x = fr * 2^ex, 0.5 <= |fr| < 1 */
    *n = (int64_t)ldexp(fr, 53);            /* exact: 53-bit significand      */
    *e = ex - 53;
    return 0;
}

uint16_t qref_rn_f16(double x)
{
    int64_t n; int e;
    if (double_split(x, &n, &e)) return isnan(x) ? 0x7E00 : (x < 0 ? 0xFC00 : 0x7C00);
    if (n == 0) return signbit(x) ? 0x8000 : 0;
    return enc_f16(rn_f16(n, e));
}

uint16_t qref_rn_bf16(double x)
{
    int64_t n; int e;
    if (double_split(x, &n, &e)) return isnan(x) ? 0x7FC0 : (x < 0 ? 0xFF80 : 0x7F80);
    if (n == 0) return signbit(x) ? 0x8000 : 0;
    return enc_bf16(rn_bf16(n, e));
}

/* binary32 rounding of a double, returned as a double (exact). */
double qref_rn_f32(double x)
{
    int64_t n; int e;
    if (double_split(x, &n, &e)) return x;
    xval v = rn_f32(n, e);
    if (v.inf) return v.inf * INFINITY;
    return ldexp((double)v.n, v.e);
}

static uint16_t enc_t(xval v, int dtype)
{
    return dtype == QREF_F16 ? enc_f16(rn_f16(v.n, v.e)) : enc_bf16(rn_bf16(v.n, v.e));
}

/* ------------------------------------------------------------------------ */
/* Field decode                                                             */
/* ------------------------------------------------------------------------ */

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* One Q4_K block (144 bytes): d, dmin, 8 scales, 8 mins, 256 codes. */
void qref_q4k_fields(const uint8_t *blk, uint16_t *d, uint16_t *dmin,
                     uint8_t sc[8], uint8_t mn[8], uint8_t q[256])
{
    const uint8_t *s12 = blk + 4, *qs = blk + 16;
    *d = rd16(blk);
    *dmin = rd16(blk + 2);
    for (int j = 0; j < 4; j++) {
        sc[j] = s12[j] & 63;
        mn[j] = s12[j + 4] & 63;
        sc[j + 4] = (uint8_t)((s12[j + 8] & 15) | ((s12[j] >> 6) << 4));
        mn[j + 4] = (uint8_t)((s12[j + 8] >> 4) | ((s12[j + 4] >> 6) << 4));
    }
    for (int g = 0; g < 4; g++)
        for (int l = 0; l < 32; l++) {
            uint8_t b = qs[32 * g + l];
            q[64 * g + l] = b & 15;
            q[64 * g + 32 + l] = b >> 4;
        }
}

/* One Q6_K block (210 bytes): 256 six-bit codes, 16 int8 scales, d. */
void qref_q6k_fields(const uint8_t *blk, uint16_t *d, int8_t s[16], uint8_t q[256])
{
    const uint8_t *ql = blk, *qh = blk + 128;
    for (int i = 0; i < 16; i++) s[i] = (int8_t)blk[192 + i];
    *d = rd16(blk + 208);
    for (int h = 0; h < 2; h++)
        for (int r = 0; r < 4; r++)
            for (int l = 0; l < 32; l++) {
                uint8_t lob = ql[64 * h + l + 32 * (r & 1)];
                int lo = (r < 2) ? (lob & 15) : (lob >> 4);
                int hi = (qh[32 * h + l] >> (2 * r)) & 3;
                q[128 * h + 32 * r + l] = (uint8_t)(lo | (hi << 4));
            }
}

/* ------------------------------------------------------------------------ */
/* Unpacked weight values                                                   */
/* ------------------------------------------------------------------------ */

/* Q4_K: factor*q - bias with factor = d*sc, bias = dmin*m, formed exactly.
 * Returns -1 if d or dmin is inf/nan. */
static int q4k_exact(uint16_t d, uint16_t dmin, int sc, int mn, int q, xval *v)
{
    int64_t nd, nm; int ed, em;
    if (f16_split(d, &nd, &ed) || f16_split(dmin, &nm, &em)) return -1;
    int e0 = ed < em ? ed : em;
    int64_t a = (nd * sc * q) * ((int64_t)1 << (ed - e0));
    int64_t b = (nm * mn) * ((int64_t)1 << (em - e0));
    xval r = {a - b, e0, 0, a < b};
    *v = r;
    return 0;
}

/* Q6_K: d*s*(q-32). */
static int q6k_exact(uint16_t d, int s, int q, xval *v)
{
    int64_t nd; int ed;
    if (f16_split(d, &nd, &ed)) return -1;
    xval r = {nd * s * (q - 32), ed, 0, 0};
    *v = r;
    return 0;
}

/* W4A16: s*(q-zp). */
static int w4_exact(uint16_t s, int q, int zp, xval *v)
{
    int64_t ns; int es;
    if (f16_split(s, &ns, &es)) return -1;
    xval r = {ns * (q - zp), es, 0, 0};
    *v = r;
    return 0;
}

/* The exact values rounded once into t. */
static int q4k_value(uint16_t d, uint16_t dmin, int sc, int mn, int q, int dtype, uint16_t *out)
{
    xval v;
    if (q4k_exact(d, dmin, sc, mn, q, &v)) return -1;
    *out = enc_t(v, dtype);
    return 0;
}

static int q6k_value(uint16_t d, int s, int q, int dtype, uint16_t *out)
{
    xval v;
    if (q6k_exact(d, s, q, &v)) return -1;
    *out = enc_t(v, dtype);
    return 0;
}

static int w4_value(uint16_t s, int q, int zp, int dtype, uint16_t *out)
{
    xval v;
    if (w4_exact(s, q, zp, &v)) return -1;
    *out = enc_t(v, dtype);
    return 0;
}

/* Scalar value of one weight for the tests (no array walk). */
int qref_q4k_weight(uint16_t d, uint16_t dmin, int sc, int mn, int q, int dtype, uint16_t *out)
{
    return q4k_value(d, dmin, sc, mn, q, dtype, out);
}
int qref_q6k_weight(uint16_t d, int s, int q, int dtype, uint16_t *out)
{
    return q6k_value(d, s, q, dtype, out);
}
int qref_w4a16_weight(uint16_t s, int q, int zp, int dtype, uint16_t *out)
{
    return w4_value(s, q, zp, dtype, out);
}

/* Whole-matrix dequant into logical W[K][N] (row k, column n). */
int qref_dequant_q4k(const uint8_t *blocks, int64_t N, int64_t K, int dtype, uint16_t *W)
{
    if (K % 256) return -2;
    int64_t nb = K / 256;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        uint16_t d, dmin;
        uint8_t sc[8], mn[8], q[256];
        for (int64_t b = 0; b < nb; b++) {
            qref_q4k_fields(blocks + (n * nb + b) * 144, &d, &dmin, sc, mn, q);
            for (int k = 0; k < 256; k++) {
                int j = k / 32;
                uint16_t w = 0;
                bad |= q4k_value(d, dmin, sc[j], mn[j], q[k], dtype, &w) != 0;
                W[(b * 256 + k) * N + n] = w;
            }
        }
    }
    return bad ? -1 : 0;
}

int qref_dequant_q6k(const uint8_t *blocks, int64_t N, int64_t K, int dtype, uint16_t *W)
{
    if (K % 256) return -2;
    int64_t nb = K / 256;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        uint16_t d;
        int8_t s[16];
        uint8_t q[256];
        for (int64_t b = 0; b < nb; b++) {
            qref_q6k_fields(blocks + (n * nb + b) * 210, &d, s, q);
            for (int k = 0; k < 256; k++) {
                uint16_t w = 0;
                bad |= q6k_value(d, s[k / 16], q[k], dtype, &w) != 0;
                W[(b * 256 + k) * N + n] = w;
            }
        }
    }
    return bad ? -1 : 0;
}

/* codes [N][K] one code per byte; scales [K/g][N] fp16 bits; zeros [K/g][N]
 * or NULL for the symmetric variant (every zero-point is 8). */
int qref_dequant_w4a16(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       int64_t N, int64_t K, int64_t group, int dtype, uint16_t *W)
{
    if (group <= 0 || K % group) return -2;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            int64_t gi = k / group;
            int zp = zeros ? zeros[gi * N + n] : 8;
            uint16_t w = 0;
            bad |= w4_value(scales[gi * N + n], codes[n * K + k], zp, dtype, &w) != 0;
            W[k * N + n] = w;
        }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* fp64 GEMM                                                                */
/* ------------------------------------------------------------------------ */

/* Y[M][N] = X[M][K] . W[K][N] in fp64 and B[M][N] = |X| . |W| (B may be NULL). */
int qref_gemm(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N, int64_t K, int dtype,
              double *Y, double *B)
{
    double *wt = (double *)malloc(sizeof(double) * (size_t)(N * K));
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
    if (!wt || !xd) { free(wt); free(xd); return -3; }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) wt[n * K + k] = t_to_double(W[k * N + n], dtype);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M * K; i++) xd[i] = t_to_double(X[i], dtype);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) {
        const double *xr = xd + m * K;
        for (int64_t n = 0; n < N; n++) {
            const double *wr = wt + n * K;
            double acc = 0.0, bnd = 0.0;
            for (int64_t k = 0; k < K; k++) {
                acc += xr[k] * wr[k];
                bnd += fabs(xr[k]) * fabs(wr[k]);
            }
            Y[m * N + n] = acc;
            if (B) B[m * N + n] = bnd;
        }
    }
    free(wt);
    free(xd);
    return 0;
}

/* The same sums for `count` chosen (row, column) pairs only. */
int qref_gemm_at(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N, int64_t K, int dtype,
                 const int64_t *rows, const int64_t *cols, int64_t count, double *Y, double *B)
{
    for (int64_t i = 0; i < count; i++)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        int64_t m = rows[i], n = cols[i];
        double acc = 0.0, bnd = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double x = t_to_double(X[m * K + k], dtype);
            double w = t_to_double(W[k * N + n], dtype);
            acc += x * w;
            bnd += fabs(x) * fabs(w);
        }
        Y[i] = acc;
        if (B) B[i] = bnd;
    }
    return 0;
}

int qref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The number of OpenMP threads the loops above use from now on (timing only:
   no result depends on it). */
void qref_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* 4. fragment-major copy: one element at a time, straight from the formula */
int qref_fragment_major(const uint16_t *X, int64_t M, int64_t K, uint16_t *out)
{
    if (M < 0 || K <= 0 || K % 128 != 0) return 1;
    const int64_t Mp = (M + 31) / 32 * 32;
    for (int64_t m = 0; m < Mp; m++)
        for (int64_t k = 0; k < K; k++) {
            const int64_t idx = ((m / 32 * (K / 128) + k / 128) * 8 + (k / 16) % 8) * 512
                                + ((k / 8) % 2 * 32 + m % 32) * 8 + k % 8;
            out[idx] = m < M ? X[m * K + k] : 0;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 5. int8-activation variant                                               */
/* ------------------------------------------------------------------------ */

/* An exact value rounded once into binary32 (never overflows here: every
 * weight is below 2^27 in magnitude). */
static float f32_of(xval v)
{
    xval r = rn_f32(v.n, v.e);
    if (r.n == 0) return v.neg ? -0.0f : 0.0f;
    return (float)ldexp((double)r.n, r.e);
}

/* Weights as binary32, logical W[K][N]: w32 = RN_f32(exact value). */
int qref_dequant_q4k_f32(const uint8_t *blocks, int64_t N, int64_t K, float *W)
{
    if (K % 256) return -2;
    int64_t nb = K / 256;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        uint16_t d, dmin;
        uint8_t sc[8], mn[8], q[256];
        for (int64_t b = 0; b < nb; b++) {
            qref_q4k_fields(blocks + (n * nb + b) * 144, &d, &dmin, sc, mn, q);
            for (int k = 0; k < 256; k++) {
                xval v = {0, 0, 0, 0};
                bad |= q4k_exact(d, dmin, sc[k / 32], mn[k / 32], q[k], &v) != 0;
                W[(b * 256 + k) * N + n] = f32_of(v);
            }
        }
    }
    return bad ? -1 : 0;
}

int qref_dequant_q6k_f32(const uint8_t *blocks, int64_t N, int64_t K, float *W)
{
    if (K % 256) return -2;
    int64_t nb = K / 256;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        uint16_t d;
        int8_t s[16];
        uint8_t q[256];
        for (int64_t b = 0; b < nb; b++) {
            qref_q6k_fields(blocks + (n * nb + b) * 210, &d, s, q);
            for (int k = 0; k < 256; k++) {
                xval v = {0, 0, 0, 0};
                bad |= q6k_exact(d, s[k / 16], q[k], &v) != 0;
                W[(b * 256 + k) * N + n] = f32_of(v);
            }
        }
    }
    return bad ? -1 : 0;
}

int qref_dequant_w4a16_f32(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                           int64_t N, int64_t K, int64_t group, float *W)
{
    if (group <= 0 || K % group) return -2;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            int64_t gi = k / group;
            int zp = zeros ? zeros[gi * N + n] : 8;
            xval v = {0, 0, 0, 0};
            bad |= w4_exact(scales[gi * N + n], codes[n * K + k], zp, &v) != 0;
            W[k * N + n] = f32_of(v);
        }
    return bad ? -1 : 0;
}

/* Nearest integer, ties to even, of a double that is an exact product. */
static double rne_int(double v)
{
    double f = floor(v), diff = v - f;  /* both exact */
    if (diff > 0.5) return f + 1.0;
    if (diff < 0.5) return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* r = RN_f32(127/amax), s = RN_f32(amax/127); both 0 when amax < 2^-96. */
static void i8_scales(double amax, float *r, float *s)
{
    if (amax < ldexp(1.0, -96)) {
        *r = 0.0f;
        *s = 0.0f;
        return;
    }
    *r = (float)(127.0 / amax);
    *s = (float)(amax / 127.0);
}

/* code = clamp(RNE_int(v * r), -127, 127); v * r is exact in binary64
 * (two binary32 significands). */
static int8_t i8_code(double v, float r)
{
    double c = rne_int(v * (double)r);
    if (c > 127.0) c = 127.0;
    if (c < -127.0) c = -127.0;
    return (int8_t)c;
}

/* Per-column scales of binary32 weights W[K][N]. */
int qref_colscale_i8(const float *W, int64_t N, int64_t K, float *r, float *s)
{
    if (N < 0 || K <= 0) return -2;
    for (int64_t n = 0; n < N; n++) {
        double amax = 0.0;
        for (int64_t k = 0; k < K; k++) amax = fmax(amax, fabs((double)W[k * N + n]));
        i8_scales(amax, &r[n], &s[n]);
    }
    return 0;
}

/* int8 weight codes Q[K][N] = RNE_int(W[k][n] * r[n]). */
int qref_requant_i8(const float *W, const float *r, int64_t N, int64_t K, int8_t *Q)
{
    if (N < 0 || K <= 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; k++)
        for (int64_t n = 0; n < N; n++) Q[k * N + n] = i8_code((double)W[k * N + n], r[n]);
    return 0;
}

/* Row quantization of X[M][K] (bit patterns of dtype): codes Q[M][K], scales s[M]. */
int qref_quant_rows_i8(const uint16_t *X, int64_t M, int64_t K, int dtype, int8_t *Q, float *s)
{
    if (M < 0 || K <= 0) return -2;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; m++) {
        double amax = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double x = t_to_double(X[m * K + k], dtype);
            bad |= !isfinite(x);
            amax = fmax(amax, fabs(x));
        }
        float r;
        i8_scales(amax, &r, &s[m]);
        for (int64_t k = 0; k < K; k++) Q[m * K + k] = i8_code(t_to_double(X[m * K + k], dtype), r);
    }
    return bad ? -1 : 0;
}

/* binary32 value -> (24-bit integer significand, exponent). */
static xval f32_split(float f)
{
    xval v = {0, 0, 0, signbit(f) != 0};
    if (f == 0.0f) return v;
    int ex;
    double fr = frexp((double)f, &ex);
    v.n = (int64_t)ldexp(fr, 24);
    v.e = ex - 24;
    return v;
}

/* Y[M][N] (bit patterns of dtype) = RN_t(RN_f32(RN_f32(acc) * RN_f32(sx[m]*sw[n]))),
 * acc = sum_k Qx[m][k] * Qw[k][n] exactly.  Qx [M][K], Qw [K][N]. */
int qref_gemm_i8(const int8_t *Qx, const float *sx, const int8_t *Qw, const float *sw,
                 int64_t M, int64_t N, int64_t K, int dtype, uint16_t *Y)
{
    if (M < 0 || N < 0 || K <= 0) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; k++) acc += (int64_t)Qx[m * K + k] * Qw[k * N + n];
            xval a = rn_f32(acc, 0);
            xval x = f32_split(sx[m]), w = f32_split(sw[n]);
            xval sc = rn_f32(x.n * w.n, x.e + w.e);
            xval y = rn_f32(a.n * sc.n, a.e + sc.e);
            Y[m * N + n] = enc_t(y, dtype);
        }
    return 0;
}

/* The int8 activation codes in the fragment-major layout (item 5). */
int qref_fragment_major_i8(const int8_t *Q, int64_t M, int64_t K, int8_t *out)
{
    if (M < 0 || K <= 0 || K % 32 != 0) return 1;
    const int64_t Mp = (M + 31) / 32 * 32;
    for (int64_t m = 0; m < Mp; m++)
        for (int64_t k = 0; k < K; k++) {
            const int64_t idx = m / 32 * 32 * K + k / 32 * 1024 + (k / 16) % 2 * 512 + m % 32 * 16 + k % 16;
            out[idx] = m < M ? Q[m * K + k] : 0;
        }
    return 0;
}
