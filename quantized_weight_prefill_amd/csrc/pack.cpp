// Host-side packers: GGUF-style k-quant blocks and GPTQ-style W4A16 fields
// -> the gfx950 panel layout described in include/qgemm.h, and back.
//
// The packing happens once per weight, off the timed path (the W4A16 PR
// repacks at load time, "Duplicate-work check").  It is pure byte and bit
// shuffling: no value is rounded or rescaled, so unpack(pack(x)) == x.
#include <cstdint>
#include <cstring>

#include "qgemm.h"

namespace {

constexpr int64_t kPanel = 16;
constexpr int64_t kQ4kBlock = 144, kQ6kBlock = 210;
constexpr int64_t kQ4kRec = 2304, kQ6kRec = 3360;

int64_t panels(int64_t N) { return (N + kPanel - 1) / kPanel; }

bool kquant_shape_ok(int64_t N, int64_t K) { return N >= 1 && K >= 256 && K % 256 == 0; }

bool w4_shape_ok(int64_t N, int64_t K, int64_t g)
{
    return N >= 1 && K >= 128 && K % 128 == 0 && g >= 32 && (g & (g - 1)) == 0 && K % g == 0;
}

// Position of code t (0..31) of a 32-code run in "pair order": word t/8,
// bit 16*(t&1) + 4*((t&7)>>1).
inline void put_nibble(uint8_t *run16, int t, uint8_t v)
{
    uint32_t w;
    std::memcpy(&w, run16 + 4 * (t / 8), 4);
    int bit = 16 * (t & 1) + 4 * ((t & 7) >> 1);
    w |= uint32_t(v & 15) << bit;
    std::memcpy(run16 + 4 * (t / 8), &w, 4);
}

inline uint8_t get_nibble(const uint8_t *run16, int t)
{
    uint32_t w;
    std::memcpy(&w, run16 + 4 * (t / 8), 4);
    int bit = 16 * (t & 1) + 4 * ((t & 7) >> 1);
    return uint8_t((w >> bit) & 15);
}

// Q6_K high pair of code t (0..31) of a run: word t/16, bit 16*(t&1) + 2*(4*u+p)
// where i = t/8, u = i&1, p = (t&7)>>1.
inline int hi_bit(int t)
{
    int i = t / 8, u = i & 1, p = (t & 7) >> 1;
    return 16 * (t & 1) + 2 * (4 * u + p);
}

inline void put_hi2(uint8_t *run8, int t, uint8_t v)
{
    uint32_t w;
    std::memcpy(&w, run8 + 4 * (t / 16), 4);
    w |= uint32_t(v & 3) << hi_bit(t);
    std::memcpy(run8 + 4 * (t / 16), &w, 4);
}

inline uint8_t get_hi2(const uint8_t *run8, int t)
{
    uint32_t w;
    std::memcpy(&w, run8 + 4 * (t / 16), 4);
    return uint8_t((w >> hi_bit(t)) & 3);
}

// GGUF Q4_K code of weight k (0..255) of a block: byte 32*(k/64) + k%32 of
// the 128-byte code field, low nibble for (k%64) < 32, high nibble otherwise.
inline int q4k_code_byte(int k) { return 32 * (k / 64) + (k % 32); }
inline int q4k_code_shift(int k) { return (k % 64) < 32 ? 0 : 4; }

// GGUF Q6_K: weight k = 128*h + 32*r + l; low nibble in ql[64h + l + 32*(r&1)]
// (low nibble for r < 2), high pair at bits 2r of qh[32h + l].
inline int q6k_ql_byte(int k) { int h = k / 128, r = (k % 128) / 32, l = k % 32; return 64 * h + l + 32 * (r & 1); }
inline int q6k_ql_shift(int k) { return ((k % 128) / 32) < 2 ? 0 : 4; }
inline int q6k_qh_byte(int k) { return 32 * (k / 128) + (k % 32); }
inline int q6k_qh_shift(int k) { return 2 * ((k % 128) / 32); }

}  // namespace

extern "C" {

size_t qgemm_q4k_packed_bytes(int64_t N, int64_t K)
{
    if (!kquant_shape_ok(N, K)) return 0;
    return size_t(panels(N) * (K / 256) * kQ4kRec);
}

size_t qgemm_q6k_packed_bytes(int64_t N, int64_t K)
{
    if (!kquant_shape_ok(N, K)) return 0;
    return size_t(panels(N) * (K / 256) * kQ6kRec);
}

size_t qgemm_w4a16_packed_bytes(int64_t N, int64_t K, int64_t g, int has_zp)
{
    if (!w4_shape_ok(N, K, g)) return 0;
    int64_t np = panels(N);
    return size_t(np * (K / 128) * 1024 + np * (K / g) * 32 + (has_zp ? np * (K / g) * 8 : 0));
}

int qgemm_q4k_pack(const void *blocks, int64_t N, int64_t K, void *out, size_t out_bytes)
{
    if (!blocks || !out) return QGEMM_ERR_NULL;
    if (!kquant_shape_ok(N, K)) return QGEMM_ERR_SHAPE;
    size_t need = qgemm_q4k_packed_bytes(N, K);
    if (out_bytes < need) return QGEMM_ERR_SIZE;
    const uint8_t *src = static_cast<const uint8_t *>(blocks);
    uint8_t *dst = static_cast<uint8_t *>(out);
    std::memset(dst, 0, need);
    const int64_t nb = K / 256;
    for (int64_t n = 0; n < N; n++) {
        const int64_t p = n / kPanel, c = n % kPanel;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = src + (n * nb + b) * kQ4kBlock;
            uint8_t *rec = dst + (p * nb + b) * kQ4kRec;
            std::memcpy(rec + 16 * c, blk, 16);  // d, dmin, 12 scale bytes
            const uint8_t *qs = blk + 16;
            for (int k = 0; k < 256; k++) {
                uint8_t v = uint8_t((qs[q4k_code_byte(k)] >> q4k_code_shift(k)) & 15);
                int h = k / 128, g = (k % 128) / 32, t = k % 32;
                put_nibble(rec + 256 + 1024 * h + (16 * g + c) * 16, t, v);
            }
        }
    }
    return QGEMM_OK;
}

int qgemm_q4k_unpack(const void *packed, int64_t N, int64_t K, void *blocks, size_t blocks_bytes)
{
    if (!packed || !blocks) return QGEMM_ERR_NULL;
    if (!kquant_shape_ok(N, K)) return QGEMM_ERR_SHAPE;
    const int64_t nb = K / 256;
    if (blocks_bytes < size_t(N * nb * kQ4kBlock)) return QGEMM_ERR_SIZE;
    const uint8_t *src = static_cast<const uint8_t *>(packed);
    uint8_t *dst = static_cast<uint8_t *>(blocks);
    for (int64_t n = 0; n < N; n++) {
        const int64_t p = n / kPanel, c = n % kPanel;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *rec = src + (p * nb + b) * kQ4kRec;
            uint8_t *blk = dst + (n * nb + b) * kQ4kBlock;
            std::memcpy(blk, rec + 16 * c, 16);
            uint8_t *qs = blk + 16;
            std::memset(qs, 0, 128);
            for (int k = 0; k < 256; k++) {
                int h = k / 128, g = (k % 128) / 32, t = k % 32;
                uint8_t v = get_nibble(rec + 256 + 1024 * h + (16 * g + c) * 16, t);
                qs[q4k_code_byte(k)] |= uint8_t(v << q4k_code_shift(k));
            }
        }
    }
    return QGEMM_OK;
}

int qgemm_q6k_pack(const void *blocks, int64_t N, int64_t K, void *out, size_t out_bytes)
{
    if (!blocks || !out) return QGEMM_ERR_NULL;
    if (!kquant_shape_ok(N, K)) return QGEMM_ERR_SHAPE;
    size_t need = qgemm_q6k_packed_bytes(N, K);
    if (out_bytes < need) return QGEMM_ERR_SIZE;
    const uint8_t *src = static_cast<const uint8_t *>(blocks);
    uint8_t *dst = static_cast<uint8_t *>(out);
    std::memset(dst, 0, need);
    const int64_t nb = K / 256;
    for (int64_t n = 0; n < N; n++) {
        const int64_t p = n / kPanel, c = n % kPanel;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = src + (n * nb + b) * kQ6kBlock;
            uint8_t *rec = dst + (p * nb + b) * kQ6kRec;
            std::memcpy(rec + 2 * c, blk + 208, 2);          // d
            std::memcpy(rec + 32 + 16 * c, blk + 192, 16);   // int8 scales
            const uint8_t *ql = blk, *qh = blk + 128;
            for (int k = 0; k < 256; k++) {
                uint8_t lo = uint8_t((ql[q6k_ql_byte(k)] >> q6k_ql_shift(k)) & 15);
                uint8_t hi = uint8_t((qh[q6k_qh_byte(k)] >> q6k_qh_shift(k)) & 3);
                int h = k / 128, g = (k % 128) / 32, t = k % 32;
                put_nibble(rec + 288 + 1024 * h + (16 * g + c) * 16, t, lo);
                put_hi2(rec + 2336 + 512 * h + (16 * g + c) * 8, t, hi);
            }
        }
    }
    return QGEMM_OK;
}

int qgemm_q6k_unpack(const void *packed, int64_t N, int64_t K, void *blocks, size_t blocks_bytes)
{
    if (!packed || !blocks) return QGEMM_ERR_NULL;
    if (!kquant_shape_ok(N, K)) return QGEMM_ERR_SHAPE;
    const int64_t nb = K / 256;
    if (blocks_bytes < size_t(N * nb * kQ6kBlock)) return QGEMM_ERR_SIZE;
    const uint8_t *src = static_cast<const uint8_t *>(packed);
    uint8_t *dst = static_cast<uint8_t *>(blocks);
    for (int64_t n = 0; n < N; n++) {
        const int64_t p = n / kPanel, c = n % kPanel;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *rec = src + (p * nb + b) * kQ6kRec;
            uint8_t *blk = dst + (n * nb + b) * kQ6kBlock;
            std::memset(blk, 0, 192);
            std::memcpy(blk + 208, rec + 2 * c, 2);
            std::memcpy(blk + 192, rec + 32 + 16 * c, 16);
            uint8_t *ql = blk, *qh = blk + 128;
            for (int k = 0; k < 256; k++) {
                int h = k / 128, g = (k % 128) / 32, t = k % 32;
                uint8_t lo = get_nibble(rec + 288 + 1024 * h + (16 * g + c) * 16, t);
                uint8_t hi = get_hi2(rec + 2336 + 512 * h + (16 * g + c) * 8, t);
                ql[q6k_ql_byte(k)] |= uint8_t(lo << q6k_ql_shift(k));
                qh[q6k_qh_byte(k)] |= uint8_t(hi << q6k_qh_shift(k));
            }
        }
    }
    return QGEMM_OK;
}

int qgemm_w4a16_pack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                     int64_t g, void *out, size_t out_bytes)
{
    if (!codes || !scales || !out) return QGEMM_ERR_NULL;
    if (!w4_shape_ok(N, K, g)) return QGEMM_ERR_SHAPE;
    const int has_zp = zeros != nullptr;
    size_t need = qgemm_w4a16_packed_bytes(N, K, g, has_zp);
    if (out_bytes < need) return QGEMM_ERR_SIZE;
    for (int64_t i = 0; i < N * K; i++)
        if (codes[i] > 15) return QGEMM_ERR_INPUT;
    if (has_zp)
        for (int64_t i = 0; i < (K / g) * N; i++)
            if (zeros[i] > 15) return QGEMM_ERR_INPUT;
    uint8_t *dst = static_cast<uint8_t *>(out);
    std::memset(dst, 0, need);
    const int64_t np = panels(N), nc = K / 128, ng = K / g;
    uint8_t *sreg = dst + np * nc * 1024;
    uint8_t *zreg = sreg + np * ng * 32;
    for (int64_t n = 0; n < N; n++) {
        const int64_t p = n / kPanel, c = n % kPanel;
        for (int64_t k = 0; k < K; k++) {
            int64_t ch = k / 128, gg = (k % 128) / 32, t = k % 32;
            put_nibble(dst + (p * nc + ch) * 1024 + (16 * gg + c) * 16, int(t), codes[n * K + k]);
        }
        for (int64_t j = 0; j < ng; j++) {
            std::memcpy(sreg + (p * ng + j) * 32 + 2 * c, &scales[j * N + n], 2);
            if (has_zp) zreg[(p * ng + j) * 8 + c / 2] |= uint8_t((zeros[j * N + n] & 15) << (4 * (c & 1)));
        }
    }
    return QGEMM_OK;
}

int qgemm_w4a16_unpack(const void *packed, int64_t N, int64_t K, int64_t g, int has_zp, uint8_t *codes,
                       uint16_t *scales, uint8_t *zeros)
{
    if (!packed || !codes || !scales || (has_zp && !zeros)) return QGEMM_ERR_NULL;
    if (!w4_shape_ok(N, K, g)) return QGEMM_ERR_SHAPE;
    const uint8_t *src = static_cast<const uint8_t *>(packed);
    const int64_t np = panels(N), nc = K / 128, ng = K / g;
    const uint8_t *sreg = src + np * nc * 1024;
    const uint8_t *zreg = sreg + np * ng * 32;
    for (int64_t n = 0; n < N; n++) {
        const int64_t p = n / kPanel, c = n % kPanel;
        for (int64_t k = 0; k < K; k++) {
            int64_t ch = k / 128, gg = (k % 128) / 32, t = k % 32;
            codes[n * K + k] = get_nibble(src + (p * nc + ch) * 1024 + (16 * gg + c) * 16, int(t));
        }
        for (int64_t j = 0; j < ng; j++) {
            std::memcpy(&scales[j * N + n], sreg + (p * ng + j) * 32 + 2 * c, 2);
            if (has_zp) zeros[j * N + n] = uint8_t((zreg[(p * ng + j) * 8 + c / 2] >> (4 * (c & 1))) & 15);
        }
    }
    return QGEMM_OK;
}

}  // extern "C"
