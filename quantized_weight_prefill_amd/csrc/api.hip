// api.hip -- host side of the fused-dequant prefill GEMM: argument checks,
// the M-ladder (which rung serves a shape), launch plans, and the C ABI of
// include/qgemm.h.  No kernels live here; the launch functions of plan.h do.
// The library holds no device memory and no mutable state: every buffer,
// the split rungs' workspace included, belongs to the caller.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>

#include "plan.h"
#include "qgemm.h"

namespace qg {
namespace {

const char *const kRungNames[RUNG_COUNT] = {"direct-small-m",    "direct-skinny-n",   "direct-wide",
                                            "mfma16-256x128",    "mfma32-128x128",    "mfma32-128x128-k2",
                                            "mfma32-128x160",    "mfma32-64x64-k4",   "mfma32-352x96",
                                            "mfma32-192x96-k2",  "mfma32-192x64-k2",  "mfma32-64x64-sk",
                                            "mfma32-64x32-k4",   "mfma32-128x64-k2",  "mfma32-96x32-k4",
                                            "mfma32-768x96",     "mfma32-512x128",    "mfma32-512x96",
                                            "mfma32-768x64-sk"};

// A one-dimensional launch of gx workgroups of `threads` threads fits when
// gx is at most 2^31-1 and the work-items along x at most 2^32-1.
bool launch_fits(long long gx, long long threads) { return gx >= 0 && gx <= INT32_MAX && gx * threads <= (long long)UINT32_MAX; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Waves splitting K inside one direct-kernel workgroup: enough waves in the
// whole grid to keep every CU streaming (about 2048), at least two chunks
// per wave, at most eight waves.  For decode-adjacent M (a pure weight
// stream) a wave keeps at least eight chunks once the grid holds 512 waves:
// with one chunk in flight ahead, shorter K ranges leave the stream idle
// while each wave starts and drains (measured at M = 1..16); with one panel
// per wave, four chunks per wave do pay while the grid stays within 2048
// waves (K = 4096, every K split forced, weights rotating: N = 4096 6.2-6.9
// against 7.7-8.3 us for four waves per workgroup, N = 2048 5.6-6.0 against
// 6.2-6.5; at N = 6144, 3072 waves, they lose by 4-10%, and with four
// panels per wave by up to 9%).
int pick_kw(long long groups, int nch, bool stream, int pn)
{
    int kw = 1;
    while (kw < 8 && groups * kw < 2048) {
        const int per = nch / (2 * kw);  // chunks per wave after doubling
        if (per < ((stream && groups * kw >= 512) ? 8 : 2) && !(stream && pn == 1 && per >= 4 && groups * 2 * kw <= 2048))
            break;
        kw *= 2;
    }
    return kw;
}

// QGEMM_OK, QGEMM_ERR_FORMAT for an unknown rung, or QGEMM_ERR_SHAPE when
// the grid would exceed what one launch can address (2^31-1 workgroups and
// 2^32-1 work-items along x, 65535 workgroups along y).
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
        if (gy > 65535 || gx > INT32_MAX) return QGEMM_ERR_SHAPE;
        pl.grid = dim3((unsigned)gx, (unsigned)gy, 1);
        break;
    }
    case RUNG_M16_256:
    case RUNG_M128:
    case RUNG_M128_K2:
    case RUNG_M128N160:
    case RUNG_M64_K4:
    case RUNG_M64_SK:
    case RUNG_M64N32_K4:
    case RUNG_M128N64_K2:
    case RUNG_M96N32_K4:
    case RUNG_M352N96:
    case RUNG_M192N96_K2:
    case RUNG_M192N64_K2:
    case RUNG_M768N96:
    case RUNG_M512N128:
    case RUNG_M512N96:
    case RUNG_M768N64_SK: {
        const bool n96 = rung == RUNG_M352N96 || rung == RUNG_M192N96_K2 || rung == RUNG_M768N96 || rung == RUNG_M512N96;
        const bool big = rung == RUNG_M768N96 || rung == RUNG_M512N128 || rung == RUNG_M512N96 ||
                         rung == RUNG_M768N64_SK;  // 8 waves, no K groups inside the workgroup
        const bool r192 = rung == RUNG_M192N96_K2 || rung == RUNG_M192N64_K2;
        const bool r64 = rung == RUNG_M64_K4 || rung == RUNG_M64_SK || rung == RUNG_M64N32_K4;
        const bool k4 = r64 || rung == RUNG_M96N32_K4;  // K split over up to four groups
        pl.rows = rung == RUNG_M16_256 ? 256 : r64 ? 64 : rung == RUNG_M352N96 ? 352 : r192 ? 192
                  : rung == RUNG_M96N32_K4 ? 96 : (rung == RUNG_M768N96 || rung == RUNG_M768N64_SK) ? 768
                  : big ? 512 : 128;
        pl.cols = rung == RUNG_M128N160 ? 160 : (rung == RUNG_M64N32_K4 || rung == RUNG_M96N32_K4) ? 32
                  : (r64 || rung == RUNG_M192N64_K2 || rung == RUNG_M128N64_K2 || rung == RUNG_M768N64_SK) ? 64
                  : n96 ? 96 : 128;
        pl.kw = ((rung == RUNG_M128_K2 || rung == RUNG_M128N64_K2 || r192) && (K / kChunk) % 2 == 0) ? 2 : 1;
        if (k4) pl.kw = (K / kChunk) % 4 == 0 ? 4 : (K / kChunk) % 2 == 0 ? 2 : 1;
        pl.waves = (rung == RUNG_M16_256 || big) ? 8 : r64 ? 2 * pl.kw : rung == RUNG_M96N32_K4 ? 3 * pl.kw
                   : rung == RUNG_M352N96 ? 11 : r192 ? 6 * pl.kw : 4 * pl.kw;
        // one-dimensional grid: the kernel renumbers tiles per XCD
        const long long tn = (np + pl.cols / 16 - 1) / (pl.cols / 16), tm = (M + pl.rows - 1) / pl.rows;
        if (!launch_fits(tn * tm, 64 * pl.waves)) return QGEMM_ERR_SHAPE;
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
        } else if (rung == RUNG_M768N64_SK) {
            // slices across workgroups: the most (up to eight) that keep the
            // grid within one round and every slice at least two chunks
            while (pl.split < 8 && tn * tm * 2 * pl.split <= kCUs && nch / (2 * pl.split) >= 2) pl.split *= 2;
        }
        if (!launch_fits(tn * tm * pl.split, 64 * pl.waves)) return QGEMM_ERR_SHAPE;
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
    pl.kw = pick_kw((long long)pl.grid.x * pl.grid.y, nch, M <= 16, pl.pn);
    pl.waves = pl.kw;
    pl.lds = pl.kw > 1 ? (size_t)pl.kw * pl.pn * pl.rb * 64 * sizeof(float) * 4 : 0;
    return launch_fits(pl.grid.x, 64 * pl.kw) ? QGEMM_OK : QGEMM_ERR_SHAPE;
}

// The M-ladder (measured on MI355X; each rung is legal for every shape):
//  * narrow N (at most four panels): the grid must run over M, so the
//    direct kernel with all panels per wave (a 128-wide tile would leave most
//    of the part idle and most of each tile padding);
//  * decode-adjacent M (at most 64 rows): each weight feeds at most 64 rows
//    and the kernel is a weight stream; up to 16 rows one panel and all rows
//    per wave (the most waves streaming, each weight unpacked once), except
//    over 1536 panels and more and, on row-major activations, at 9..16 rows
//    over 512 panels and more: four panels and 16 rows per wave; 17..64 rows
//    over at most 256 panels one panel and all rows per wave (on row-major
//    activations above 32 rows 16 rows and four panels per wave), or on
//    fragment-major activations 64x64 tiles with K split across workgroups
//    too (split_pays); over more panels the direct kernels up to 32 rows
//    (four panels and all rows per wave from 512 panels, for fp16 Q4_K up to
//    48 rows), above that the round model's streaming tiles;
//  * above 64 rows, the round model of round_model_rung over the direct
//    kernels and the streaming tiles that run one workgroup per CU (64x32,
//    96x32 and 64x64 with K split four ways, 128x64 and 192x64 with K split
//    two ways), whenever its cheapest rung is one of those and not one of the
//    large tiles below;
//  * the 8-wave 256x128 tile on 16x16x32 MFMAs (each weight unpacked once
//    for 256 rows) when the occupancy model below has it finish no later
//    than the 128-row tiles;
//  * at most 256 tiles of 128x128 over K >= 8192: the 128x128 tile on
//    32x32x16 MFMAs with K split between two wave groups;
//  * otherwise the 128-row tile on 32x32x16 MFMAs, 128 or 160 columns wide,
//    whichever the occupancy model below finishes first.
// On fragment-major activations the large tiles instead go by their
// full-round costs (large_tile_xf): the three-waves-per-SIMD tiles (192x64
// and 192x96 with K split over two 6-wave groups, 352x96), the K-split
// 128x128, 256x128, 128x128 and 128x160 tiles and the 8-wave tiles of 64-
// and 96-row waves (512x96, 512x128, 768x96), whichever finishes its whole
// rounds first.  Row-major Q6_K, which has no 160-wide tile, takes the
// 352x96 tile by the occupancy rule, one round of 192x96 tiles where the
// 256-row tile would serve, and the 256-row tile from 512 of its tiles.
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

// The split rung at 33..64 rows over 129..256 panels (N = 2049..4096) on
// fragment-major activations: one panel and all rows per wave reads the
// activations once per panel, the 64x64 tiles split across workgroups read a
// slice of them.  Measured on MI355X (weights rotating), K = 12288 (four
// slices): Q6_K and W4A16, and every format in bf16, from 33 rows (Q6_K M =
// 64 24.2 against 28.1 us; W4A16 M = 48 18.5 against 20.4), fp16 Q4_K at
// 49..64 only.  Shorter K leaves too few chunks per slice.  (Above 64 rows
// the round model's tiles beat it on fragment-major activations; on
// row-major ones it would win at 65..128 rows over N <= 4096, by 3-25%, but
// the row-major ladder serves the format entry points, which take no
// workspace.)
bool split_pays(int fmt, int dtype, long long M, long long np, long long K, int xl)
{
    const long long nch = K / kChunk;
    if (xl != X_FRAG || np > 256 || np <= 128 || M > 64) return false;
    if (nch < 64 || nch % 16 != 0) return false;
    if (dtype == DT_BF16 || fmt != FMT_Q4K) return M > 32;
    return M > 48;
}

// Cost of one full round of a rung's workgroups (256 CUs, `per_cu`
// workgroups on each at once), in microseconds at K = 4096, by activation
// layout (row-major, fragment-major) and format (Q4_K, Q6_K, W4A16); the
// direct kernels have a row per number of 16-row blocks each wave carries
// (`rb`, as make_plan sets it; 0 for the streaming tiles).  Measured on
// MI355X with every rung forced, weights rotating through 320 MB: medians of
// time / rounds, scaled to K = 4096, over M = 17..512, N = 1024..27648 and K
// = 4096..14336, both dtypes (the four-panel direct kernel runs 10-20%
// faster in fp16 on Q4_K and has rows per dtype; its 48-row variant spills
// for Q6_K and W4A16, and the zero entries leave it out for them, as they
// leave out the 192x64 tile on row-major activations, where it never wins).
// `large` marks the tiles whose rules follow in select_rung: above 64 rows,
// when one of them is cheapest, the model defers to those.
struct RoundCost {
    int rung, rb, per_cu, dtype, large;  // dtype -1: both
    float us[2][3];
};
constexpr RoundCost kRoundCost[] = {
    {RUNG_M64_K4, 0, 1, -1, 0, {{21.4f, 23.8f, 20.7f}, {16.4f, 18.7f, 15.2f}}},
    {RUNG_M64N32_K4, 0, 1, -1, 0, {{18.2f, 19.7f, 17.7f}, {9.7f, 11.0f, 8.6f}}},
    {RUNG_M96N32_K4, 0, 1, -1, 0, {{25.1f, 26.9f, 24.6f}, {13.0f, 14.9f, 12.4f}}},
    {RUNG_M128N64_K2, 0, 1, -1, 0, {{31.5f, 33.3f, 30.7f}, {19.5f, 21.1f, 18.4f}}},
    {RUNG_M192N64_K2, 0, 1, -1, 0, {{0.0f, 0.0f, 0.0f}, {25.2f, 27.6f, 24.2f}}},
    {RUNG_SMALL_M, 2, 1, -1, 0, {{8.0f, 8.4f, 7.8f}, {5.5f, 5.8f, 5.0f}}},
    {RUNG_SMALL_M, 3, 1, -1, 0, {{12.1f, 12.8f, 12.0f}, {7.0f, 7.9f, 6.7f}}},
    {RUNG_SMALL_M, 4, 1, -1, 0, {{15.5f, 15.9f, 15.4f}, {7.4f, 7.7f, 6.8f}}},
    {RUNG_SKINNY_N, 1, 1, -1, 0, {{11.0f, 12.5f, 9.7f}, {10.6f, 12.0f, 9.2f}}},
    {RUNG_WIDE, 2, 1, DT_F16, 0, {{13.8f, 16.3f, 13.3f}, {11.9f, 14.9f, 11.5f}}},
    {RUNG_WIDE, 3, 1, DT_F16, 0, {{17.8f, 0.0f, 0.0f}, {14.1f, 0.0f, 0.0f}}},
    {RUNG_WIDE, 2, 1, DT_BF16, 0, {{14.4f, 15.7f, 12.8f}, {13.3f, 13.9f, 10.5f}}},
    {RUNG_WIDE, 3, 1, DT_BF16, 0, {{20.4f, 0.0f, 0.0f}, {16.6f, 0.0f, 0.0f}}},
    {RUNG_M128_K2, 0, 1, -1, 1, {{36.3f, 40.2f, 34.8f}, {33.1f, 37.2f, 31.5f}}},
    {RUNG_M128, 0, 2, -1, 1, {{38.1f, 41.9f, 36.3f}, {38.2f, 41.4f, 35.0f}}},
    {RUNG_M128N160, 0, 2, -1, 1, {{49.7f, 90.7f, 46.5f}, {52.0f, 91.7f, 47.6f}}},
    {RUNG_M16_256, 0, 1, -1, 1, {{54.2f, 58.4f, 52.6f}, {48.9f, 51.9f, 48.0f}}},
    {RUNG_M192N96_K2, 0, 1, -1, 1, {{50.2f, 52.2f, 48.4f}, {32.1f, 34.2f, 30.4f}}},
};

// The rung the round model finishes first; above 64 rows -1 when that is
// one of the large tiles.  On a tie the earlier entry of the table, a
// streaming tile before a direct kernel (Q4_K at M = 100, N = 5120, K =
// 13824, bf16: 64x64 tiles 46.0 against 54.5 us for direct-wide, whose
// costs tie).  A K-split tile takes part only with an even chunk count:
// with an odd one it runs a single K group.  With two chunks over (K =
// 11008: 86 chunks) the four-way tiles run two K groups and measured no
// slower per round than with four (64x32 tiles at M = 100, N = 4096: 44-50
// us, the K = 12288 times scaled to that K).  Measured against the fastest
// forced rung over the sweeps the table comes from: 1.002-1.007 of it on
// average, and 1.010-1.014 on shapes outside them (hidden sizes 5120,
// 11008, 13824, 14336, 27648); the earlier fixed thresholds came to
// 1.06-1.13 there.  E.g. M = 320, N = 1024 on fragment-major Q4_K: 64x32
// tiles 10.5 against 17.1 us for direct-wide; M = 129..192, N = 4096: 96x32
// tiles 13.8-14.9 against 17.2-18.8; M = 320..512, N = 4096: 128x64 tiles
// 22.7-26.0 against 28.0-32.5 for 192x64; M = 65..128, N = 12288: 128x64
// tiles 0.58-0.86 of the former time; M = 40..64, N = 6144: 64x32 tiles
// 0.6-0.7 of the time of one panel per wave; row-major M = 48..64, N =
// 1024..4096: 16 rows and four panels per wave 0.57-0.72 of the time of
// one panel and all rows per wave.
int round_model_rung(int fmt, long long M, long long N, long long K, int xl, int dtype)
{
    double best = 1e30;
    int pick = -1, large = 1;
    for (const RoundCost &rc : kRoundCost) {
        const float us = rc.us[xl == X_FRAG][fmt];
        if ((rc.dtype >= 0 && rc.dtype != dtype) || us <= 0.0f) continue;
        Plan pl;
        if (make_plan(rc.rung, M, N, K, pl) != QGEMM_OK || pl.rb != rc.rb) continue;
        if (pl.kw == 1 && rc.rb == 0 && rc.rung != RUNG_M128 && rc.rung != RUNG_M128N160 && rc.rung != RUNG_M16_256)
            continue;  // a K-split tile left with one K group
        const long long wgs = (long long)pl.grid.x * pl.grid.y * pl.grid.z;
        const long long per_round = (long long)kCUs * rc.per_cu;
        const double cost = us * (double)((wgs + per_round - 1) / per_round);
        if (cost < best) {
            best = cost;
            pick = rc.rung;
            large = rc.large;
        }
    }
    return large && M > 64 ? -1 : pick;
}

// Full-round cost of the large tiles on fragment-major activations, in
// microseconds at K = 4096 per format (Q4_K, Q6_K, W4A16): medians of time /
// rounds over the shapes whose last round is at least 75% full, every large
// tile forced on M = 384..4096, N = 4096..24576, K = 4096 and 12288 (fp16,
// weights rotating).  A round is 256 workgroups (512 for the 4-wave 128x128
// and 128x160 tiles, two per CU).  The 8-wave tiles of 64- and 96-row waves
// cost the most per round but unpack each weight once for 512 or 768 rows
// and read a third to a half of the LDS bytes per MFMA.
struct LargeCost {
    int rung, per_cu;
    float us[3];
};
constexpr LargeCost kLargeCostXf[] = {
    {RUNG_M192N64_K2, 1, {31.8f, 34.5f, 31.0f}}, {RUNG_M128_K2, 1, {41.2f, 46.0f, 40.0f}},
    {RUNG_M192N96_K2, 1, {42.8f, 46.4f, 42.0f}}, {RUNG_M16_256, 1, {61.6f, 65.6f, 61.6f}},
    {RUNG_M352N96, 1, {70.1f, 75.0f, 69.5f}},    {RUNG_M128, 2, {71.4f, 81.6f, 69.8f}},
    {RUNG_M128N160, 2, {94.9f, 129.2f, 92.2f}},  {RUNG_M512N96, 1, {96.3f, 100.4f, 95.8f}},
    {RUNG_M512N128, 1, {104.4f, 109.0f, 104.1f}}, {RUNG_M768N96, 1, {137.5f, 145.0f, 135.1f}},
};

// The large tile with the fewest modelled microseconds on fragment-major
// activations (whole rounds times the round cost; a K-split tile left with
// one K group takes no part; ties to the earlier entry).  Against the
// fastest forced rung over that sweep: 1.004 of it on average, where the
// rule chain it replaces came to 1.056 (e.g. M = 640, N = 24576: 768x96
// 139 against 175 us for 256x128; M = 1024, N = 12288: 512x96 102 against
// 119 us for 128x128; Q6_K at M = 640, N = 12288: 352x96 80 against 122 us).
int large_tile_xf(int fmt, long long M, long long N, long long K)
{
    double best = 1e30;
    int pick = RUNG_M128;
    for (const LargeCost &lc : kLargeCostXf) {
        Plan pl;
        if (make_plan(lc.rung, M, N, K, pl) != QGEMM_OK) continue;
        const bool ksplit = lc.rung == RUNG_M192N64_K2 || lc.rung == RUNG_M128_K2 || lc.rung == RUNG_M192N96_K2;
        if (ksplit && pl.kw == 1) continue;
        const long long wgs = (long long)pl.grid.x * pl.grid.y * pl.grid.z, per_round = (long long)kCUs * lc.per_cu;
        const double cost = lc.us[fmt] * (double)((wgs + per_round - 1) / per_round) * (double)K / 4096.0;
        if (cost < best) {
            best = cost;
            pick = lc.rung;
        }
    }
    return pick;
}

// The 768x64 tiles with K split across workgroups, on fragment-major
// activations (the caller passes the partial sums' workspace): for 513..768
// rows of Q4_K or Q6_K over at least 96 chunks (K >= 12288), when 64-column
// tiles times a power-of-two slice count of 2..8 make exactly one round.
// Each weight is then unpacked once for all the rows and the CUs stay busy
// although the tiles alone would fill a quarter or half of them.  Measured
// against the ladder's choice (fp16, weights rotating, interleaved): Q6_K
// 658x12288 -> 4096 92.0 against 101.4 us (four slices), 520 rows 86.7 against
// 93.2, 768 rows 95.6 against 103.5, K = 16384 115.2 against 132.9, N = 8192
// at 600 rows 159.1 against 183.7 (two slices); Q4_K 658x12288 -> 4096 89.2
// against 95.2, -> 2048 53.4 against 57.7 (eight slices).  It loses at K =
// 8192 (Q4_K, 700 rows: 68.0 against 64.2 us) and at 400 rows (80.8 against
// 71.9), where the 768-row tile is half empty.
bool split768_pays(int fmt, long long M, long long np, long long K)
{
    if (fmt == FMT_W4 || M <= 512 || M > 768 || K / kChunk < 96 || np % 4 != 0) return false;
    const long long tn = np / 4;
    for (long long S = 2; S <= 8; S *= 2)
        if (tn * S == kCUs) return true;
    return false;
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
        // 17..64 rows: the split rung where split_pays, else the round model
        // over the direct kernels and the streaming tiles (on row-major
        // activations above 32 rows over few panels 16 rows and four panels
        // per wave, over 384 panels 64x32 tiles in one round, over 768 64x64
        // tiles in one round, over 1536 the K-split 128x128 tile ...)
        if (split_pays(fmt, dtype, M, np, K, xl)) return RUNG_M64_SK;
        return round_model_rung(fmt, M, N, K, xl, dtype);
    }
    if (xl == X_FRAG && split768_pays(fmt, M, np, K)) return RUNG_M768N64_SK;
    if (const int r = round_model_rung(fmt, M, N, K, xl, dtype); r >= 0) return r;
    if (xl == X_FRAG) return large_tile_xf(fmt, M, N, K);
    // row-major activations: the rule chain below (its tiles read 32 rows x
    // 32 bytes per activation operand, so the three-waves-per-SIMD and
    // 8-wave tiles that win on fragment-major activations lose here, except
    // the ones named)
    const long long t128 = tn * ((M + 127) / 128), t256 = tn * ((M + 255) / 256);
    // occupancy model: a 256x128 tile counts as two 128x128 tiles; the
    // 128-row rungs as stream_cost has them (160 wide only off Q6_K)
    const double c256 = 2.0 * (double)((t256 + kCUs - 1) / kCUs);
    const double c128 = std::min(stream_cost(M, np, 128), fmt != FMT_Q6K ? stream_cost(M, np, 160) : 1e30);
    const long long r192 = (M + 191) / 192, t192 = r192 * ((np + 5) / 6);
    // Q6_K, which has no 160-wide tile: the 352x96 tile (11 waves, three per
    // SIMD) when its rounds, each costing 1.22 rounds of the 256-row tile,
    // come out cheapest (M = 700, N = 11008..24576: 101-204 against 130-222
    // us for 128x128; the other formats' 128x160 tile beats it there)
    if (fmt == FMT_Q6K) {
        const long long t352 = ((np + 5) / 6) * ((M + 351) / 352);
        const double c352 = 2.44 * (double)((t352 + kCUs - 1) / kCUs);
        if (c352 < c256 && c352 < c128) return RUNG_M352N96;
    }
    // the 256-row tile when the occupancy model has it finish no later than
    // the 128-row tiles (it unpacks each weight once for 256 rows); Q6_K
    // takes one round of 192x96 K-split tiles instead where they fit (M =
    // 300..384, N = 11008..12288: 61-66 against 73-76 us; for the other
    // formats, and elsewhere, they lose by 5-50%), and the 256-row tile also
    // from 512 of its tiles (M = 1500..4096, N = 11008..24576: 0.88-0.98 of
    // the 128x128 time; at 1.5 rounds, 384 tiles, it loses by 6-9%)
    if (c256 <= c128 && fmt == FMT_Q6K && (K / kChunk) % 2 == 0 && r192 * 192 <= (M + 127) / 128 * 128 && t192 <= kCUs)
        return RUNG_M192N96_K2;
    if (c256 <= c128 || (fmt == FMT_Q6K && t256 >= 512)) return RUNG_M16_256;
    // few tiles: split K inside the workgroup, over a long K only, where the
    // halves' activation reloads stay affordable
    if (t128 <= 256 && K >= 8192) return RUNG_M128_K2;
    // 160-wide tiles when they even out the tiles per CU (Q6_K's larger raw
    // runs do not fit that variant's registers)
    if (fmt != FMT_Q6K && stream_cost(M, np, 160) < stream_cost(M, np, 128)) return RUNG_M128N160;
    return RUNG_M128;
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

// Bytes of the split rungs' partial sums: S slices of 4-byte sums (fp32 or
// int32), each row-major [M][N], the slice stride rounded up to 4 elements
// so that every slice starts 16-byte aligned.  0 for the other rungs.
size_t split_ws_bytes(const Plan &pl, long long M, long long N)
{
    if (pl.split <= 1 && pl.rung != RUNG_M64_SK && pl.rung != RUNG_M768N64_SK) return 0;
    const long long stride = (M * N + 3) & ~3LL;
    return (size_t)(stride * pl.split) * 4;
}

// K split across workgroups: the slices' partial sums go to the caller's
// workspace, then one launch adds them in slice order and rounds once.
int gemm_split(int fmt, int dtype, int xl, const Plan &pl, Args a, void *ws, hipStream_t s)
{
    const long long MN = (long long)a.M * a.N, stride = (MN + 3) & ~3LL;
    a.part = (float *)ws;
    a.pstride = stride;
    a.split = pl.split;
    hipError_t e = launch(fmt, dtype, xl, pl, a, s);
    if (e == hipSuccess) e = launch_splitk_reduce(dtype, (const float *)ws, a.Y, MN, stride, pl.split, s);
    return launch_status(e, kRungNames[pl.rung]);
}

// Checks shared by the GEMM entry points; on success fills the plan.
int gemm_plan(int fmt, int rung, long long M, long long N, long long K, long long group, int dtype, int xl, Plan &pl)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, M, N, K, group);
    if (st != QGEMM_OK) return st;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (rung < -1 || rung >= RUNG_COUNT) return QGEMM_ERR_FORMAT;
    return make_plan(rung < 0 ? select_rung(fmt, M > 0 ? M : 1, N, K, xl, dtype) : rung, M > 0 ? M : 1, N, K, pl);
}

// Every check of a GEMM call but the workspace's: QGEMM_OK with the plan and
// the workspace bytes it needs, or the first error (M == 0 is QGEMM_OK with
// no launch to make).
int gemm_args(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
              long long group, int dtype, int xl, Plan &pl, size_t &need)
{
    need = 0;
    int st = gemm_plan(fmt, rung, M, N, K, group, dtype, xl, pl);
    if (st != QGEMM_OK || M == 0) return st;
    if (!X || !W || !Y) return QGEMM_ERR_NULL;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return QGEMM_ERR_ALIGN;
    need = split_ws_bytes(pl, M, N);
    return QGEMM_OK;
}

int gemm(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
         long long group, int has_zp, int dtype, void *ws, size_t ws_bytes, void *stream, int xl = X_ROW)
{
    Plan pl;
    size_t need = 0;
    int st = gemm_args(fmt, rung, X, W, Y, M, N, K, group, dtype, xl, pl, need);
    if (st != QGEMM_OK || M == 0) return st;
    if (need > 0) {
        if (!ws || ws_bytes < need) return QGEMM_ERR_SIZE;
        if (!aligned16(ws)) return QGEMM_ERR_ALIGN;
        if (!launch_fits(((M * N + 3) / 4 + 255) / 256, 256)) return QGEMM_ERR_SHAPE;
    }
    Args a = make_args(fmt, X, W, Y, M, N, K, group, has_zp);
    a.kw = pl.kw;
    if (need > 0) return gemm_split(fmt, dtype, xl, pl, a, ws, (hipStream_t)stream);
    return launch_status(launch(fmt, dtype, xl, pl, a, (hipStream_t)stream), kRungNames[pl.rung]);
}

long long packed_bytes(int fmt, long long N, long long K, long long group, int has_zp)
{
    if (fmt == FMT_Q4K) return (long long)qgemm_q4k_packed_bytes(N, K);
    if (fmt == FMT_Q6K) return (long long)qgemm_q6k_packed_bytes(N, K);
    return (long long)qgemm_w4a16_packed_bytes(N, K, group, has_zp);
}

// Grouped plan.  Up to 16 rows per expert on average (ceil(T/E)), or when
// the grid is too small to fill the chip without splitting K (the direct
// plan's kw above 1), the direct grouped kernel: four panels per wave, one
// or two 16-row blocks, K split as the direct rungs split it.  Otherwise the
// shared-activation kernel, 32-row tiles up to 48 rows per expert and
// 80-row tiles above.  Measured on the 128-expert, 8-per-token routing of a
// 658-token prompt (Zipf-like counts) with the counts scaled to 10-288 rows
// per expert, Q4_K 2048 -> 768 and Q6_K 768 -> 2048, weights rotating: at
// 10 rows the two kernels tie (38 against 38 us, 47 against 48); at 41 rows
// the shared kernel takes 58-60 against the direct kernel's 63-67 us and
// 70-72 against 71-77; from 66 rows its 80-row tiles beat 64x64 streaming
// tiles (two 32-row waves, weights unpacked once into LDS) by 12-25% (288
// rows: 200-204 against 250-258 us, 235 against 305-320).  32-row tiles lead up to 49 rows
// (Q4_K), 48- to 96-row tiles differ by a few percent from 49 to 99 rows,
// and 80-row tiles lead or tie from 99 rows on; a wider wave (four panels)
// or eight waves measured slower throughout.
Plan grouped_plan(long long T, long long E, long long N, long long K)
{
    Plan pl{};
    const long long np = (N + 15) / 16, avg = (T + E - 1) / E;
    pl.rung = GROUPED_DIRECT;
    pl.pn = 4;
    pl.rb = avg <= 16 ? 1 : 2;
    pl.grid = dim3((unsigned)ceil_div(np, 4), (unsigned)(ceil_div(T, 16 * pl.rb) + E), 1);
    pl.kw = pick_kw((long long)pl.grid.x * pl.grid.y, (int)(K / kChunk), false, pl.pn);
    pl.waves = pl.kw;
    pl.rows = 16 * pl.rb;
    pl.cols = 64;
    pl.lds = pl.kw > 1 ? (size_t)pl.kw * pl.pn * pl.rb * 64 * sizeof(float) * 4 : 0;
    if (avg > 16 && pl.kw == 1) {
        pl.rung = GROUPED_SHARED;
        pl.pn = 2;
        pl.rb = avg <= 48 ? 2 : 5;
        pl.waves = 4;
        pl.grid = dim3((unsigned)ceil_div(np, 8), (unsigned)(ceil_div(T, 16 * pl.rb) + E), 1);
        pl.rows = 16 * pl.rb;
        pl.cols = 128;
        pl.lds = 0;
    }
    return pl;
}

int grouped(int fmt, const void *X, const void *W, void *Y, const int32_t *offs, long long E, long long T, long long N,
            long long K, long long group, int has_zp, int dtype, void *stream, int xl)
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
    const Plan pl = grouped_plan(T, E, N, K);
    if (!launch_fits(pl.grid.x, 64 * pl.waves)) return QGEMM_ERR_SHAPE;
    a.kw = pl.kw;
    return launch_status(launch_grouped(fmt, dtype, xl, pl, a, (hipStream_t)stream), "grouped");
}

size_t staged_scratch_bytes(long long N, long long K)
{
    if (N < 1 || K < 1 || K % kChunk != 0 || N > INT32_MAX || K > INT32_MAX) return 0;
    return (size_t)((N + 15) / 16) * 16 * (size_t)K * 2;
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
    if (!launch_fits((((N + 15) / 16) * (K / kChunk) * 64 + 255) / 256, 256)) return QGEMM_ERR_SHAPE;
    Args a = make_args(fmt, X, W, Y, M, N, K, group, has_zp);
    return launch_status(launch_staged(fmt, dtype, a, (uint8_t *)scratch, pl, (hipStream_t)stream), "staged");
}

// ---------------------------------------------------------------------------
// int8-activation path: rungs, validation, launches.
// ---------------------------------------------------------------------------

const char *const kI8RungNames[I8_RUNG_COUNT] = {"i8-128x128",   "i8-256x128",   "i8-128x128-k2",
                                                   "i8-256x96",    "i8-512x96",    "i8-352x96",
                                                   "i8-192x96-k2", "i8-192x64-k2", "i8-64x64-sk",
                                                   "i8-768x96"};
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
    case I8_M768N96: pl.rows = 768; pl.cols = 96; pl.waves = 8; break;
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
    if (!launch_fits(tn * tm, 64 * pl.waves)) return QGEMM_ERR_SHAPE;
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
    if (!launch_fits(tn * tm * pl.split, 64 * pl.waves)) return QGEMM_ERR_SHAPE;
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
//  * otherwise the 256x128, 256x96, 352x96, 512x96 or 768x96 tile,
//    whichever finishes in the fewest rounds of one workgroup per CU, a
//    round costing 1, 0.85, 1.17, 1.35 and 2.1 (fitted to the measured
//    times: the merged gate_up at M = 658 91 us on 352x96 against 107 on
//    256x96 and 117 on 256x128, and 93.7 on one round of 768x96 against
//    95.0 on two of 352x96; M = 2048 121 us on 512x96 against 133 on
//    256x128 and 138 on 352x96; M = 4096 238 against 260 and 268).  The
//    352-row tile runs three waves per SIMD and unpacks each weight for 352
//    rows: two of its row tiles cover M = 658 where 256-row tiles need
//    three; the 768-row tile unpacks each weight once for 768 rows.
int i8_select(int fmt, long long M, long long N, long long K)
{
    const long long np = (N + 15) / 16, t128 = ((M + 127) / 128) * ((np + 7) / 8), r192 = (M + 191) / 192;
    const long long nch = K / kChunk;
    // few 64x64 tiles: those tiles with K split across workgroups as well,
    // every format and M, up to 96 tiles (128 for Q6_K, whose unpack weighs
    // most: M = 128, N = 4096 23.7 against 26.4 us), and up to 256 over K >=
    // 8192
    // (every rung forced, weights rotating: up to 64 tiles 0.44-0.66 of the
    // time of the 192x64 K-split tile, e.g. Q4_K 4096->1024 at M = 128..256
    // 11.7-13.1 against 20.2-20.8 us, Q6_K 12288->4096 at M = 16..128
    // 24.9-35.8 against 56.1-59.5; 96 tiles 0.82-0.97; at K = 12288 256
    // tiles 0.85-0.91; at K = 4096 from 128 tiles a tie, from 256 a loss of
    // 7-15%)
    const long long t64 = ((np + 3) / 4) * ((M + 63) / 64);
    if (nch % 8 == 0 && nch >= 16 && (t64 <= (fmt == FMT_Q6K ? 128 : 96) || (nch >= 64 && t64 <= 256)))
        return I8_M64_SK;
    if ((K / kChunk) % 2 == 0 && r192 * ((np + 3) / 4) <= kCUs) return I8_M192N64_K2;
    if ((K / kChunk) % 2 == 0 && r192 * ((np + 5) / 6) <= kCUs) return I8_M192N96_K2;
    if (t128 <= 256 && (K / kChunk) % 2 == 0) return I8_M128_K2;
    if (M <= 128) return I8_M128;
    const long long tm256 = (M + 255) / 256, tm352 = (M + 351) / 352, tm512 = (M + 511) / 512, tm768 = (M + 767) / 768;
    const long long tn128 = (np + 7) / 8, tn96 = (np + 5) / 6;
    const auto rounds = [](long long tiles) { return (double)((tiles + kCUs - 1) / kCUs); };
    // (the 768-row tile of 96-row waves, a round costing 2.1: one round of it
    // for the merged gate_up at M = 658, 93.7 against 95.0 us for two of
    // 352x96, Q6_K 104.2 against 117.8; M = 1500, N = 12288: 100.1 against
    // 116.8 us for three rounds of 256x96)
    const double c[5] = {rounds(tm256 * tn128), 0.85 * rounds(tm256 * tn96), 1.17 * rounds(tm352 * tn96),
                         1.35 * rounds(tm512 * tn96), 2.1 * rounds(tm768 * tn96)};
    const int rung[5] = {I8_M256, I8_M256N96, I8_M352N96, I8_M512N96, I8_M768N96};
    int best = 0;
    for (int i = 1; i < 5; i++)
        if (c[i] < c[best]) best = i;
    return rung[best];
}

template <int DT>
hipError_t launch_i8_dt(int fmt, const Plan &pl, const Args &a, hipStream_t s)
{
    if (fmt == FMT_Q4K) return launch_i8_fd<FMT_Q4K, DT>(pl, a, s);
    if (fmt == FMT_Q6K) return launch_i8_fd<FMT_Q6K, DT>(pl, a, s);
    return launch_i8_fd<FMT_W4, DT>(pl, a, s);
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int i8_gemm_plan(int fmt, int rung, long long M, long long N, long long K, long long group, int dtype, Plan &pl)
{
    if (fmt == FMT_W4 && group == 0) return QGEMM_ERR_FORMAT;
    int st = check_shape(fmt, M, N, K, group);
    if (st != QGEMM_OK) return st;
    if (K > kI8MaxK) return QGEMM_ERR_SHAPE;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (rung < -1 || rung >= I8_RUNG_COUNT) return QGEMM_ERR_FORMAT;
    const long long m = M > 0 ? M : 1;
    return i8_plan(rung < 0 ? i8_select(fmt, m, N, K) : rung, m, N, K, pl);
}

size_t i8_ws_bytes(const Plan &pl, long long M, long long N)
{
    if (pl.rung != I8_M64_SK) return 0;
    return (size_t)(((M * N + 3) & ~3LL) * pl.split) * 4;
}

int i8_gemm(int fmt, int rung, const void *Xq, const float *sx, const void *W, const float *rw, const float *sw,
            void *Y, long long M, long long N, long long K, long long group, int has_zp, int dtype, void *ws,
            size_t ws_bytes, void *stream)
{
    Plan pl;
    int st = i8_gemm_plan(fmt, rung, M, N, K, group, dtype, pl);
    if (st != QGEMM_OK) return st;
    if (M == 0) return QGEMM_OK;
    if (!Xq || !sx || !W || !rw || !sw || !Y) return QGEMM_ERR_NULL;
    if (!aligned16(Xq) || !aligned16(W) || !aligned16(Y) || !aligned4(sx) || !aligned4(rw) || !aligned4(sw))
        return QGEMM_ERR_ALIGN;
    Args a = make_args(fmt, Xq, W, Y, M, N, K, group, has_zp);
    a.sx = sx;
    a.rw = rw;
    a.sw = sw;
    const hipStream_t s = (hipStream_t)stream;
    const size_t need = i8_ws_bytes(pl, M, N);
    if (need > 0) {
        // int32 partial sums per K slice in the caller's workspace, then
        // their exact total through the unsplit epilogue
        if (!ws || ws_bytes < need) return QGEMM_ERR_SIZE;
        if (!aligned16(ws)) return QGEMM_ERR_ALIGN;
        const long long MN = M * N, stride = (MN + 3) & ~3LL;
        if (!launch_fits(((MN + 3) / 4 + 255) / 256, 256)) return QGEMM_ERR_SHAPE;
        a.part = (float *)ws;
        a.pstride = stride;
        a.split = pl.split;
        hipError_t e = dtype == DT_F16 ? launch_i8_dt<DT_F16>(fmt, pl, a, s) : launch_i8_dt<DT_BF16>(fmt, pl, a, s);
        if (e == hipSuccess) e = launch_i8_reduce(dtype, (const int *)ws, sx, sw, (uint16_t *)Y, (int)M, (int)N, stride, pl.split, s);
        return launch_status(e, kI8RungNames[pl.rung]);
    }
    const hipError_t e = dtype == DT_F16 ? launch_i8_dt<DT_F16>(fmt, pl, a, s) : launch_i8_dt<DT_BF16>(fmt, pl, a, s);
    return launch_status(e, kI8RungNames[pl.rung]);
}

int i8_quantize(const void *X, void *Xq, float *sx, long long M, long long K, int dtype, void *stream)
{
    // one wave per padded row, four per workgroup of 256 threads
    if (M < 0 || K < 32 || K % 32 != 0 || M > INT32_MAX - 31 || K > INT32_MAX) return QGEMM_ERR_SHAPE;
    if (!launch_fits((M + 31) / 32 * 8, 256)) return QGEMM_ERR_SHAPE;
    if (dtype != DT_F16 && dtype != DT_BF16) return QGEMM_ERR_DTYPE;
    if (M == 0) return QGEMM_OK;
    if (!X || !Xq || !sx) return QGEMM_ERR_NULL;
    if (!aligned16(X) || !aligned16(Xq) || !aligned4(sx)) return QGEMM_ERR_ALIGN;
    return launch_status(launch_i8_quant(dtype, (const uint16_t *)X, (uint8_t *)Xq, sx, (int)M, (int)K, (hipStream_t)stream),
                         "i8 quantize");
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
    return launch_status(launch_i8_colscale(fmt, a, rw, sw, (hipStream_t)stream), "i8 colscale");
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

int gemm_check(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
               long long group, int dtype, int xl, size_t *ws_need)
{
    Plan pl;
    return gemm_args(fmt, rung, X, W, Y, M, N, K, fmt == FMT_W4 ? group : 0, dtype, xl, pl, *ws_need);
}

int gemm_entry(int fmt, int rung, const void *X, const void *W, void *Y, long long M, long long N, long long K,
               long long group, int has_zp, int dtype, void *ws, size_t ws_bytes, void *stream, int xl)
{
    return gemm(fmt, rung, X, W, Y, M, N, K, fmt == FMT_W4 ? group : 0, has_zp, dtype, ws, ws_bytes, stream, xl);
}

}  // namespace qg

using namespace qg;

extern "C" {

const char *qgemm_status_str(int status)
{
    switch (status) {
    case QGEMM_OK: return "ok";
    case QGEMM_ERR_NULL: return "null pointer";
    case QGEMM_ERR_SHAPE: return "illegal shape";
    case QGEMM_ERR_DTYPE: return "unsupported dtype";
    case QGEMM_ERR_ALIGN: return "pointer not aligned";
    case QGEMM_ERR_FORMAT: return "unsupported format, group size or rung";
    case QGEMM_ERR_SIZE: return "buffer too small";
    case QGEMM_ERR_HIP: return "HIP launch failed";
    case QGEMM_ERR_INPUT: return "malformed input data";
    default: return "unknown status";
    }
}

// The format entry points use the row-major ladder, which never picks a rung
// that needs a workspace (a CPU test sweeps it); were it to, the call would
// fail with QGEMM_ERR_SIZE rather than allocate.
int qgemm_q4k(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int dtype, void *stream)
{
    return gemm(FMT_Q4K, -1, X, W, Y, M, N, K, 0, 0, dtype, nullptr, 0, stream);
}

int qgemm_q6k(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int dtype, void *stream)
{
    return gemm(FMT_Q6K, -1, X, W, Y, M, N, K, 0, 0, dtype, nullptr, 0, stream);
}

int qgemm_w4a16(const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K, int64_t group_size,
                int has_zp, int dtype, void *stream)
{
    return gemm(FMT_W4, -1, X, W, Y, M, N, K, group_size, has_zp, dtype, nullptr, 0, stream);
}

int qgemm_gemm_rung(int format, int rung, const void *X, const void *W, void *Y, int64_t M, int64_t N, int64_t K,
                    int64_t group_size, int has_zp, int dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm(format, rung, X, W, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, workspace,
                workspace_bytes, stream);
}

size_t qgemm_workspace_bytes(int format, int rung, int layout, int64_t M, int64_t N, int64_t K, int dtype)
{
    if (layout != QGEMM_X_ROW && layout != QGEMM_X_FRAG) return 0;
    Plan pl;
    if (gemm_plan(format, rung, M, N, K, format == FMT_W4 ? 128 : 0, dtype, layout, pl) != QGEMM_OK) return 0;
    return M > 0 ? split_ws_bytes(pl, M, N) : 0;
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
    if (!launch_fits(((M + 31) / 32) * (K / kChunk), 256)) return QGEMM_ERR_SHAPE;
    if (M == 0) return QGEMM_OK;
    if (!X || !Xf) return QGEMM_ERR_NULL;
    if (!aligned16(X) || !aligned16(Xf)) return QGEMM_ERR_ALIGN;
    return launch_status(launch_x_to_xf((const uint16_t *)X, (uint16_t *)Xf, (int)M, (int)K, (hipStream_t)stream),
                         "x_to_xf");
}

int qgemm_gemm_xf(int format, int rung, const void *Xf, const void *W, void *Y, int64_t M, int64_t N, int64_t K,
                  int64_t group_size, int has_zp, int dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm(format, rung, Xf, W, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, workspace,
                workspace_bytes, stream, X_FRAG);
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
    if (!launch_fits(((long long)a.np * (K / kChunk) * 64 + 255) / 256, 256)) return QGEMM_ERR_SHAPE;
    return launch_status(launch_dequant(format, dtype, a, (uint16_t *)Wout, (hipStream_t)stream), "dequant");
}

size_t qgemm_staged_scratch_bytes(int64_t N, int64_t K) { return staged_scratch_bytes(N, K); }

int qgemm_staged(int format, const void *X, const void *Wpacked, void *scratch, size_t scratch_bytes, void *Y, int64_t M,
                 int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream)
{
    return staged(format, X, Wpacked, scratch, scratch_bytes, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype,
                  stream);
}

int qgemm_grouped(int format, const void *X, const void *Wpacked, void *Y, const int32_t *offsets, int64_t E, int64_t T,
                  int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream)
{
    return grouped(format, X, Wpacked, Y, offsets, E, T, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, stream,
                   X_ROW);
}

int qgemm_grouped_xf(int format, const void *Xf, const void *Wpacked, void *Y, const int32_t *offsets, int64_t E,
                     int64_t T, int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream)
{
    return grouped(format, Xf, Wpacked, Y, offsets, E, T, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype, stream,
                   X_FRAG);
}

int qgemm_grouped_plan(int64_t T, int64_t E, int64_t N, int64_t K, int32_t *info8)
{
    if (!info8) return QGEMM_ERR_NULL;
    if (T < 0 || E < 1 || E > INT32_MAX / 2 || N < 1 || N > INT32_MAX || K < kChunk || K % kChunk != 0 ||
        K > INT32_MAX || T > INT32_MAX || (long long)ceil_div(T, 16) + E > 65535)
        return QGEMM_ERR_SHAPE;
    const Plan pl = grouped_plan(T, E, N, K);
    const int32_t v[8] = {pl.rung, pl.rows, pl.cols, pl.waves, pl.kw, (int32_t)pl.grid.x, (int32_t)pl.grid.y, 0};
    for (int i = 0; i < 8; i++) info8[i] = v[i];
    return QGEMM_OK;
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
                  void *workspace, size_t workspace_bytes, void *stream)
{
    return i8_gemm(format, rung, Xq, sx, Wpacked, rw, sw, Y, M, N, K, format == FMT_W4 ? group_size : 0, has_zp, dtype,
                   workspace, workspace_bytes, stream);
}

size_t qgemm_i8_workspace_bytes(int format, int rung, int64_t M, int64_t N, int64_t K)
{
    Plan pl;
    if (i8_gemm_plan(format, rung, M, N, K, format == FMT_W4 ? 128 : 0, DT_F16, pl) != QGEMM_OK) return 0;
    return M > 0 ? i8_ws_bytes(pl, M, N) : 0;
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
