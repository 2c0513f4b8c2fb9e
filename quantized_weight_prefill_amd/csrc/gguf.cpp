// gguf.cpp -- a reader for the GGUF container (version 2 and 3), the file
// format of the k-quant checkpoints the batched-prefill post runs (a Q4_K_M
// Qwen3-8B: Q4_K for most projections, Q6_K for ffn_down and attn_v).  The
// caller hands over the whole file as one host buffer (read or memory-mapped);
// every function walks it in place, allocates nothing and checks every
// length, count and offset against the buffer before using it, so a
// truncated or malformed file is an error, never a read out of bounds.
//
// Layout (little-endian throughout):
//   u32 magic "GGUF", u32 version, u64 tensor count, u64 metadata count;
//   metadata: string key, u32 value type, value;
//   tensor infos: string name, u32 n_dims, u64 dims[n_dims] (dims[0] the row
//   length, contiguous in memory), u32 ggml type, u64 offset into the data
//   section;
//   padding to `general.alignment` (default 32), then the data section.
// A string is u64 length + bytes (no terminator); an array is u32 element
// type, u64 count, the elements.
#include <cstdint>
#include <cstring>

#include "qgemm.h"

namespace {

enum : uint32_t {
    T_U8 = 0, T_I8 = 1, T_U16 = 2, T_I16 = 3, T_U32 = 4, T_I32 = 5, T_F32 = 6, T_BOOL = 7,
    T_STRING = 8, T_ARRAY = 9, T_U64 = 10, T_I64 = 11, T_F64 = 12
};
constexpr uint32_t kMagic = 0x46554747u;  // "GGUF"
constexpr int kMaxDims = 4;

struct Cursor {
    const uint8_t *p;
    uint64_t size, pos;
    bool ok;
    bool need(uint64_t n)
    {
        if (!ok || n > size - pos) ok = false;
        return ok;
    }
    template <typename T>
    T get()
    {
        T v{};
        if (need(sizeof(T))) {
            std::memcpy(&v, p + pos, sizeof(T));
            pos += sizeof(T);
        }
        return v;
    }
    void skip(uint64_t n)
    {
        if (need(n)) pos += n;
    }
    // a string: its bytes at *s, length *n (not terminated)
    void str(const char **s, uint64_t *n)
    {
        const uint64_t len = get<uint64_t>();
        *n = len;
        *s = ok && need(len) ? (const char *)(p + pos) : nullptr;
        if (ok) pos += len;
    }
};

uint64_t scalar_bytes(uint32_t t)
{
    switch (t) {
    case T_U8: case T_I8: case T_BOOL: return 1;
    case T_U16: case T_I16: return 2;
    case T_U32: case T_I32: case T_F32: return 4;
    case T_U64: case T_I64: case T_F64: return 8;
    default: return 0;
    }
}

// Skips one value of type t (nested arrays are not part of the format).
void skip_value(Cursor &c, uint32_t t, int depth = 0)
{
    if (const uint64_t b = scalar_bytes(t)) {
        c.skip(b);
    } else if (t == T_STRING) {
        const char *s;
        uint64_t n;
        c.str(&s, &n);
    } else if (t == T_ARRAY && depth == 0) {
        const uint32_t et = c.get<uint32_t>();
        const uint64_t n = c.get<uint64_t>();
        if (const uint64_t b = scalar_bytes(et)) {
            if (n > (c.size - c.pos) / b) c.ok = false;
            else c.skip(n * b);
        } else if (et == T_STRING) {
            for (uint64_t i = 0; i < n && c.ok; i++) skip_value(c, T_STRING, 1);
        } else {
            c.ok = false;
        }
    } else {
        c.ok = false;
    }
}

struct Header {
    uint32_t version;
    uint64_t n_tensors, n_kv;
    uint64_t alignment;
    uint64_t infos;   // offset of the first tensor info
    uint64_t data;    // offset of the data section
};

// Bytes per block and weights per block of the ggml types this library
// reads tensor sizes for (0: unknown type).
void type_block(uint32_t type, uint64_t *block_bytes, uint64_t *block_elems)
{
    *block_bytes = 0;
    *block_elems = 1;
    switch (type) {
    case 0: *block_bytes = 4; break;      // F32
    case 1: *block_bytes = 2; break;      // F16
    case 30: *block_bytes = 2; break;     // BF16
    case 2: *block_bytes = 18; *block_elems = 32; break;   // Q4_0
    case 3: *block_bytes = 20; *block_elems = 32; break;   // Q4_1
    case 6: *block_bytes = 22; *block_elems = 32; break;   // Q5_0
    case 7: *block_bytes = 24; *block_elems = 32; break;   // Q5_1
    case 8: *block_bytes = 34; *block_elems = 32; break;   // Q8_0
    case 10: *block_bytes = 84; *block_elems = 256; break;  // Q2_K
    case 11: *block_bytes = 110; *block_elems = 256; break; // Q3_K
    case QGEMM_GGML_Q4_K: *block_bytes = 144; *block_elems = 256; break;
    case 13: *block_bytes = 176; *block_elems = 256; break; // Q5_K
    case QGEMM_GGML_Q6_K: *block_bytes = 210; *block_elems = 256; break;
    default: break;
    }
}

int read_header(const void *buf, size_t size, Header &h)
{
    if (!buf) return QGEMM_ERR_NULL;
    Cursor c{(const uint8_t *)buf, (uint64_t)size, 0, true};
    const uint32_t magic = c.get<uint32_t>();
    h.version = c.get<uint32_t>();
    if (!c.ok || magic != kMagic || (h.version != 2 && h.version != 3)) return QGEMM_ERR_INPUT;
    h.n_tensors = c.get<uint64_t>();
    h.n_kv = c.get<uint64_t>();
    if (!c.ok || h.n_tensors > size || h.n_kv > size) return QGEMM_ERR_INPUT;
    h.alignment = 32;
    for (uint64_t i = 0; i < h.n_kv && c.ok; i++) {
        const char *key;
        uint64_t klen;
        c.str(&key, &klen);
        const uint32_t t = c.get<uint32_t>();
        if (!c.ok) break;
        if (klen == 17 && std::memcmp(key, "general.alignment", 17) == 0 && t == T_U32) {
            const uint32_t a = c.get<uint32_t>();
            if (a == 0 || (a & (a - 1)) != 0) return QGEMM_ERR_INPUT;
            h.alignment = a;
        } else {
            skip_value(c, t);
        }
    }
    if (!c.ok) return QGEMM_ERR_INPUT;
    h.infos = c.pos;
    for (uint64_t i = 0; i < h.n_tensors && c.ok; i++) {
        const char *name;
        uint64_t nlen;
        c.str(&name, &nlen);
        const uint32_t nd = c.get<uint32_t>();
        if (nd == 0 || nd > kMaxDims) return QGEMM_ERR_INPUT;
        c.skip(8ull * nd + 4 + 8);
    }
    if (!c.ok) return QGEMM_ERR_INPUT;
    const uint64_t data = (c.pos + h.alignment - 1) / h.alignment * h.alignment;
    if (data > size) return QGEMM_ERR_INPUT;
    h.data = data;
    return QGEMM_OK;
}

struct TensorInfo {
    const char *name;
    uint64_t name_len;
    uint32_t n_dims, type;
    uint64_t dims[kMaxDims];
    uint64_t offset;  // absolute, in the buffer
    uint64_t bytes;
};

int tensor_info(const void *buf, size_t size, int64_t index, TensorInfo &ti)
{
    Header h;
    int st = read_header(buf, size, h);
    if (st != QGEMM_OK) return st;
    if (index < 0 || (uint64_t)index >= h.n_tensors) return QGEMM_ERR_SHAPE;
    Cursor c{(const uint8_t *)buf, (uint64_t)size, h.infos, true};
    for (int64_t i = 0; i <= index; i++) {
        c.str(&ti.name, &ti.name_len);
        ti.n_dims = c.get<uint32_t>();
        if (!c.ok || ti.n_dims == 0 || ti.n_dims > kMaxDims) return QGEMM_ERR_INPUT;
        for (uint32_t d = 0; d < ti.n_dims; d++) ti.dims[d] = c.get<uint64_t>();
        ti.type = c.get<uint32_t>();
        ti.offset = c.get<uint64_t>();
    }
    if (!c.ok) return QGEMM_ERR_INPUT;
    for (uint32_t d = ti.n_dims; d < kMaxDims; d++) ti.dims[d] = 1;
    uint64_t bb, be;
    type_block(ti.type, &bb, &be);
    // element count and byte size, without overflow
    uint64_t n = 1;
    for (int d = 0; d < kMaxDims; d++) {
        if (ti.dims[d] == 0) return QGEMM_ERR_INPUT;
        if (n > UINT64_MAX / ti.dims[d]) return QGEMM_ERR_INPUT;
        n *= ti.dims[d];
    }
    ti.bytes = 0;
    if (bb) {
        if (ti.dims[0] % be != 0) return QGEMM_ERR_INPUT;  // rows are whole blocks
        const uint64_t blocks = n / be;
        if (blocks > UINT64_MAX / bb) return QGEMM_ERR_INPUT;
        ti.bytes = blocks * bb;
    }
    if (ti.offset % h.alignment != 0 || ti.offset > size - h.data) return QGEMM_ERR_INPUT;
    ti.offset += h.data;
    if (ti.bytes > size - ti.offset) return QGEMM_ERR_INPUT;
    return QGEMM_OK;
}

}  // namespace

extern "C" {

int qgemm_gguf_header(const void *buf, size_t size, uint32_t *version, int64_t *n_tensors, int64_t *n_kv,
                      int64_t *alignment, int64_t *data_offset)
{
    Header h;
    const int st = read_header(buf, size, h);
    if (st != QGEMM_OK) return st;
    if (version) *version = h.version;
    if (n_tensors) *n_tensors = (int64_t)h.n_tensors;
    if (n_kv) *n_kv = (int64_t)h.n_kv;
    if (alignment) *alignment = (int64_t)h.alignment;
    if (data_offset) *data_offset = (int64_t)h.data;
    return QGEMM_OK;
}

int qgemm_gguf_tensor_info(const void *buf, size_t size, int64_t index, char *name, size_t name_cap, int32_t *type,
                           int32_t *n_dims, int64_t *dims4, int64_t *data_offset, int64_t *data_bytes)
{
    TensorInfo ti;
    const int st = tensor_info(buf, size, index, ti);
    if (st != QGEMM_OK) return st;
    if (name && name_cap > 0) {
        const uint64_t n = ti.name_len < name_cap - 1 ? ti.name_len : name_cap - 1;
        std::memcpy(name, ti.name, n);
        name[n] = '\0';
        if (ti.name_len >= name_cap) return QGEMM_ERR_SIZE;
    }
    if (type) *type = (int32_t)ti.type;
    if (n_dims) *n_dims = (int32_t)ti.n_dims;
    if (dims4)
        for (int d = 0; d < kMaxDims; d++) dims4[d] = ti.dims[d] > (uint64_t)INT64_MAX ? -1 : (int64_t)ti.dims[d];
    if (data_offset) *data_offset = (int64_t)ti.offset;
    if (data_bytes) *data_bytes = (int64_t)ti.bytes;
    return QGEMM_OK;
}

int qgemm_gguf_find_kv(const void *buf, size_t size, const char *key, int32_t *value_type, int64_t *value_offset,
                       int64_t *value_bytes)
{
    if (!buf || !key) return QGEMM_ERR_NULL;
    Header h;
    int st = read_header(buf, size, h);
    if (st != QGEMM_OK) return st;
    const size_t want = std::strlen(key);
    Cursor c{(const uint8_t *)buf, (uint64_t)size, 24, true};
    for (uint64_t i = 0; i < h.n_kv && c.ok; i++) {
        const char *k;
        uint64_t klen;
        c.str(&k, &klen);
        const uint32_t t = c.get<uint32_t>();
        const uint64_t start = c.pos;
        skip_value(c, t);
        if (!c.ok) break;
        if (klen == want && std::memcmp(k, key, want) == 0) {
            if (value_type) *value_type = (int32_t)t;
            if (value_offset) *value_offset = (int64_t)start;
            if (value_bytes) *value_bytes = (int64_t)(c.pos - start);
            return QGEMM_OK;
        }
    }
    return c.ok ? QGEMM_ERR_FORMAT : QGEMM_ERR_INPUT;
}

size_t qgemm_gguf_packed_bytes(const void *buf, size_t size, int64_t index)
{
    TensorInfo ti;
    if (tensor_info(buf, size, index, ti) != QGEMM_OK || ti.n_dims != 2) return 0;
    if (ti.dims[0] > INT64_MAX || ti.dims[1] > INT64_MAX) return 0;
    if (ti.type == QGEMM_GGML_Q4_K) return qgemm_q4k_packed_bytes((int64_t)ti.dims[1], (int64_t)ti.dims[0]);
    if (ti.type == QGEMM_GGML_Q6_K) return qgemm_q6k_packed_bytes((int64_t)ti.dims[1], (int64_t)ti.dims[0]);
    return 0;
}

int qgemm_gguf_pack(const void *buf, size_t size, int64_t index, void *out, size_t out_bytes, int32_t *format,
                    int64_t *N, int64_t *K)
{
    TensorInfo ti;
    const int st = tensor_info(buf, size, index, ti);
    if (st != QGEMM_OK) return st;
    if (ti.type != QGEMM_GGML_Q4_K && ti.type != QGEMM_GGML_Q6_K) return QGEMM_ERR_FORMAT;
    if (ti.n_dims != 2 || ti.dims[0] > INT32_MAX || ti.dims[1] > INT32_MAX) return QGEMM_ERR_SHAPE;
    const int64_t k = (int64_t)ti.dims[0], n = (int64_t)ti.dims[1];
    if (format) *format = ti.type == QGEMM_GGML_Q4_K ? QGEMM_FMT_Q4K : QGEMM_FMT_Q6K;
    if (N) *N = n;
    if (K) *K = k;
    if (!out) return QGEMM_ERR_NULL;
    const uint8_t *blocks = (const uint8_t *)buf + ti.offset;
    return ti.type == QGEMM_GGML_Q4_K ? qgemm_q4k_pack(blocks, n, k, out, out_bytes)
                                      : qgemm_q6k_pack(blocks, n, k, out, out_bytes);
}

}  // extern "C"
