/*
 * qgemm.h -- C ABI of the MI355X (gfx950) fused-dequant prefill linear layer
 *
 *     Y[M,N] = X[M,K] . dequant(W)[K,N]
 *
 * W is stored compressed: GGUF-style Q4_K or Q6_K super-blocks, or W4A16
 * (4-bit codes with a group-wise fp16 scale and 4-bit zero-point).  The
 * kernels read every packed weight byte from HBM once per output tile,
 * unpack it in registers and feed it to fp16/bf16 MFMA with fp32
 * accumulation; no dequantized copy of W is ever written to memory.
 *
 * The pages cited below, by the short names used in this file:
 *   the batched-prefill post  "How ZINC's RDNA4 batched prefill went from 42
 *                             to 208 tok/s" (ZINC blog)
 *   the W4A16 PR              "[ROCm][Perf] W4A16: packed fp16 prefill
 *                             dequant" (vLLM pull request 55711)
 *   the delta-net page        "Delta-Net: llama.cpp vs ZINC Analysis" (ZINC docs)
 *   the dequant-scratch post  "The dequant scratch round-trip is ZINC's last
 *                             RDNA4 prefill tax" (ZINC blog)
 *   the sparkinfer PR         sparkinfer pull request 511 (chunk-parallel GDN
 *                             scan, int8 prefill GEMM, skinny GEMM)
 * The dequant-scratch post, "The two passes hiding inside one matmul", is the
 * method: the fused form moves 0.5625 bytes per Q4_K weight instead of 4.5625.
 *
 * Conventions for every entry point
 *   - Plain pointers and sizes only.  Device pointers must come from the HIP
 *     allocator of the current device; host pointers are ordinary memory.
 *     The caller owns every buffer, including the workspace of the rungs that
 *     split K across workgroups.  The library never synchronises the stream,
 *     never allocates device memory and keeps no mutable global state, so
 *     every call is re-entrant; calls that share a workspace buffer must be
 *     ordered (one stream), as for any buffer both write.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GEMM and dequant calls are asynchronous on that stream.
 *   - dtype: QGEMM_F16 or QGEMM_BF16.  X and Y have that type; the weights are
 *     unpacked into it (the MFMA operand type).
 *   - X is row-major [M][K] contiguous, Y is row-major [M][N] contiguous.
 *     X, Y and Wpacked must be 16-byte aligned; Y must not alias X or W.
 *   - Return value: QGEMM_OK (0) or a negative status.  Argument errors are
 *     found before any launch and leave Y untouched; a shape whose grid would
 *     not fit one launch (more than 2^31-1 workgroups or 2^32-1 threads along
 *     x, or 65535 row groups of a direct rung along y) is QGEMM_ERR_SHAPE,
 *     and the M-ladder never picks a rung it cannot launch.  A failed launch
 *     returns QGEMM_ERR_HIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation, as with any HIP launch.  An unsupported format or
 *     dtype is an error, never a silent fallback (the batched-prefill post,
 *     "Bug 2: Q6_K had a gate but no dispatcher").
 *
 * Unpacked weight values (bit-exact contract)
 *   Q4_K : w = RN_t( d*sc*q - dmin*m )      (sc, m: 6-bit; q: 4-bit)
 *   Q6_K : w = RN_t( d*s*(q - 32) )         (s: int8 per 16; q: 6-bit)
 *   W4A16: w = RN_t( s*(q - zp) )           (zp = 8 when has_zp == 0)
 *   RN_t is one round-to-nearest-even of the exact value into fp16/bf16 (the
 *   W4A16 PR, "1. Packed fp16 dequant": the subtraction is exact and the
 *   multiply that follows rounds once; the k-quants' factor*q - bias is the
 *   batched-prefill post's, "The fix: K-parallel batched DMMV").  The
 *   products are accumulated in fp32; the order of that accumulation is
 *   unspecified (it depends on the rung; the W4A16 PR, "Model evaluation").
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define QGEMM_OK 0
#define QGEMM_ERR_NULL (-1)   /* a required pointer is NULL                  */
#define QGEMM_ERR_SHAPE (-2)  /* M < 0, N < 1, K not a legal multiple, ...   */
#define QGEMM_ERR_DTYPE (-3)  /* dtype is not QGEMM_F16 / QGEMM_BF16         */
#define QGEMM_ERR_ALIGN (-4)  /* a pointer is not 16-byte aligned            */
#define QGEMM_ERR_FORMAT (-5) /* unknown format, group size or rung          */
#define QGEMM_ERR_SIZE (-6)   /* an output buffer is too small               */
#define QGEMM_ERR_HIP (-7)    /* the HIP launch failed                       */
#define QGEMM_ERR_INPUT (-8)  /* malformed input data (e.g. code above 15)   */

/* Human-readable text for a status code (static storage, never NULL).  Every
 * failure names itself instead of degrading to another path (the
 * batched-prefill post, "Bug 2: Q6_K had a gate but no dispatcher": an
 * unsupported quant type surfaced as an error, not as a wrong answer). */
const char *qgemm_status_str(int status);

/* ---- enumerations -------------------------------------------------------- */
#define QGEMM_F16 0
#define QGEMM_BF16 1

#define QGEMM_FMT_Q4K 0
#define QGEMM_FMT_Q6K 1
#define QGEMM_FMT_W4A16 2

/* activation layouts (qgemm_workspace_bytes): row-major X, or the
 * fragment-major copy of qgemm_x_to_xf */
#define QGEMM_X_ROW 0
#define QGEMM_X_FRAG 1

/* ---- packed layout (what the packers write and the kernels read) --------
 *
 * Output columns are grouped in panels of 16; Np = ceil(N/16).  Columns past
 * N inside the last panel are zero-filled and never stored to Y.  Inside a
 * panel everything is arranged so that one wave's 64 lanes x 16-byte loads
 * cover 1 KB of contiguous memory, and each lane's 16 bytes are the 32 codes
 * of one (column, 32-wide K run): the codes of one sub-block.
 *
 * "Pair order" of a 16-byte code run (32 codes, k = k0 .. k0+31): 32-bit word
 * i holds codes k0+8i .. k0+8i+7; code k0+8i+2p sits at bits [4p, 4p+4) and
 * code k0+8i+2p+1 at bits [16+4p, 20+4p), p = 0..3 (the ExLlama shuffle of
 * the W4A16 PR, "1. Packed fp16 dequant": one mask yields both halves of an
 * fp16 pair).
 *
 * Q4_K: one 2304-byte record per (panel p, super-block b), record index
 *   p*(K/256) + b.  Bytes [0,256): the 16 columns' block headers (fp16 d,
 *   fp16 dmin, the 12 bytes of 6-bit scales/mins, exactly as in the GGUF
 *   block), column c at 16*c.  Bytes [256,2304): codes, half h (k 128h ..
 *   128h+127 of the block) at 256 + 1024*h, then sub-block g of that half and
 *   column c at (16*g + c)*16, in pair order.          (144 bytes / 256 w)
 * Q6_K: one 3360-byte record per (panel, super-block).  [0,32): the fp16 d
 *   of columns 0..15; [32,288): their 16 int8 scales (16 bytes per column);
 *   [288,2336): low code nibbles laid out as the Q4_K codes; [2336,3360):
 *   high 2-bit pairs, half h at 2336 + 512*h, sub-block g and column c at
 *   (16*g + c)*8: two 32-bit words, word e for codes k0+16e .. k0+16e+15;
 *   code k0+8i+2p+t (i = 2e+u, t = 0/1) has its top two bits at bit
 *   16*t + 2*(4u+p) of word e.                          (210 bytes / 256 w)
 * W4A16: codes first: one 1024-byte run per (panel, 128-wide K chunk),
 *   index p*(K/128) + c, group g and column c at (16*g + c)*16, pair order.
 *   Then fp16 scales [Np][K/group][16], then (has_zp only) zero-points
 *   [Np][K/group][8 bytes], column c in the nibble c (low nibble first).
 */

/* ---- host-side packers (host memory in, host memory out) -----------------
 * Run once per weight at load time, off the GEMM path (the W4A16 PR repacks
 * at load, "Duplicate-work check"; the bytes per weight are the
 * dequant-scratch post's 0.5625 for Q4_K, "The two passes hiding inside one
 * matmul").
 * blocks: [N][K/256] GGUF-style blocks, column n's blocks contiguous along K
 * (Q4_K: 144 B = fp16 d, fp16 dmin, 12 B scales/mins, 128 B codes; Q6_K:
 * 210 B = 128 B ql, 64 B qh, 16 B int8 scales, fp16 d).  K % 256 == 0.
 * *_packed_bytes returns 0 for an illegal shape.  pack returns
 * QGEMM_ERR_SIZE when out_bytes is smaller than *_packed_bytes and
 * QGEMM_ERR_NULL for a NULL buffer.  unpack is the exact inverse (for tests
 * and for exporting packed weights); pack and unpack are pure byte shuffles
 * and never touch a value. */
size_t qgemm_q4k_packed_bytes(int64_t N, int64_t K);
int qgemm_q4k_pack(const void *blocks, int64_t N, int64_t K, void *out, size_t out_bytes);
int qgemm_q4k_unpack(const void *packed, int64_t N, int64_t K, void *blocks, size_t blocks_bytes);

/* Q6_K: the format of ffn_down and attn_v in a Q4_K_M checkpoint (the
 * batched-prefill post, "Bug 2: Q6_K had a gate but no dispatcher"); same
 * conventions as the Q4_K packer above. */
size_t qgemm_q6k_packed_bytes(int64_t N, int64_t K);
int qgemm_q6k_pack(const void *blocks, int64_t N, int64_t K, void *out, size_t out_bytes);
int qgemm_q6k_unpack(const void *packed, int64_t N, int64_t K, void *blocks, size_t blocks_bytes);

/* W4A16 (GPTQ-style, the W4A16 PR, "1. Packed fp16 dequant"): codes [N][K],
 * one 4-bit code (0..15) per byte; scales [K/group][N] fp16 bits; zeros
 * [K/group][N] (0..15) or NULL for the symmetric variant (zero-point 8, and
 * then no zero-point bytes are stored).  K % 128 == 0, group a power of two
 * of at least 32, K % group == 0 (a 32-wide run never straddles a group: the
 * W4A16 PR, "2. dtype-aware gfx1151 tile selection").  Codes or zeros above
 * 15 give QGEMM_ERR_INPUT. */
size_t qgemm_w4a16_packed_bytes(int64_t N, int64_t K, int64_t group_size, int has_zp);
int qgemm_w4a16_pack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                     int64_t group_size, void *out, size_t out_bytes);
int qgemm_w4a16_unpack(const void *packed, int64_t N, int64_t K, int64_t group_size, int has_zp, uint8_t *codes,
                       uint16_t *scales, uint8_t *zeros);

/* ---- GGUF checkpoints (host memory) ----------------------------------------
 * The k-quant weights the pages run come in GGUF files: the batched-prefill
 * post's Qwen3-8B Q4_K_M ("The measured result"), whose ffn_down and attn_v
 * tensors are Q6_K and the rest Q4_K ("Bug 2: Q6_K had a gate but no
 * dispatcher").  These calls read such a file -- version 2 or 3 of the
 * container: header, metadata, tensor infos, the data section at
 * `general.alignment` (default 32) -- from one caller-owned host buffer
 * holding the whole file (read or memory-mapped), allocate nothing, and
 * check every length, count and offset against `size`: a truncated or
 * malformed file returns QGEMM_ERR_INPUT, never a read outside the buffer.
 * A tensor's dims[0] is its row length (contiguous in the file): for a
 * linear layer's weight, dims = {K, N}, which is the packers' [N][K/256]
 * block order, so a Q4_K or Q6_K tensor packs with no reordering.
 *
 * qgemm_gguf_header: the container version, tensor and metadata counts, the
 *   alignment and the byte offset of the data section.
 * qgemm_gguf_tensor_info: tensor `index` (0 .. n_tensors-1; else
 *   QGEMM_ERR_SHAPE): its name (NUL-terminated into name[name_cap];
 *   QGEMM_ERR_SIZE, with the name cut, when it does not fit), ggml type
 *   (QGEMM_GGML_Q4_K, QGEMM_GGML_Q6_K, ...), dimension count and dims (dims4[4],
 *   1 past n_dims), the byte offset of its data in the buffer and its byte
 *   size (0 for a type this library does not size).  Any output may be NULL.
 * qgemm_gguf_find_kv: the metadata entry `key` (NUL-terminated): its value
 *   type (the container's codes: 4 u32, 6 f32, 8 string, 9 array, ...), and
 *   the byte offset and size of its encoded value in the buffer (a string:
 *   u64 length then bytes; an array: u32 element type, u64 count, elements);
 *   QGEMM_ERR_FORMAT when no entry has that key.
 * qgemm_gguf_packed_bytes / qgemm_gguf_pack: a two-dimensional Q4_K or Q6_K
 *   tensor packed with qgemm_q4k_pack / qgemm_q6k_pack into `out` (host,
 *   caller-owned, at least qgemm_gguf_packed_bytes bytes); *format (QGEMM_FMT_*),
 *   *N = dims[1] and *K = dims[0] say how to call the GEMMs on it.  Any other
 *   tensor type is QGEMM_ERR_FORMAT (packed_bytes returns 0), never a
 *   conversion. */
#define QGEMM_GGML_Q4_K 12
#define QGEMM_GGML_Q6_K 14
int qgemm_gguf_header(const void *buf, size_t size, uint32_t *version, int64_t *n_tensors, int64_t *n_kv,
                      int64_t *alignment, int64_t *data_offset);
int qgemm_gguf_tensor_info(const void *buf, size_t size, int64_t index, char *name, size_t name_cap, int32_t *type,
                           int32_t *n_dims, int64_t *dims4, int64_t *data_offset, int64_t *data_bytes);
int qgemm_gguf_find_kv(const void *buf, size_t size, const char *key, int32_t *value_type, int64_t *value_offset,
                       int64_t *value_bytes);
size_t qgemm_gguf_packed_bytes(const void *buf, size_t size, int64_t index);
int qgemm_gguf_pack(const void *buf, size_t size, int64_t index, void *out, size_t out_bytes, int32_t *format,
                    int64_t *N, int64_t *K);

/* ---- fused-dequant GEMMs (device memory, asynchronous on `stream`) ------- */

/* Q4_K weights (the dequant-scratch post, "What removing it was worth": the
 * Q4_K dequant fused into the matrix-core GEMM; the batched-prefill post,
 * "The fix: K-parallel batched DMMV").  K % 256 == 0, M >= 0 (M == 0 is a
 * no-op), N >= 1.  Row-major X; the rung comes from the row-major M-ladder,
 * which never picks a rung that needs a workspace. */
int qgemm_q4k(const void *X, const void *Wpacked, void *Y, int64_t M, int64_t N, int64_t K, int dtype,
              void *stream);

/* Q6_K weights (the batched-prefill post, "Bug 2: Q6_K had a gate but no
 * dispatcher": ffn_down / attn_v of a Q4_K_M checkpoint).  Same
 * preconditions as qgemm_q4k. */
int qgemm_q6k(const void *X, const void *Wpacked, void *Y, int64_t M, int64_t N, int64_t K, int dtype,
              void *stream);

/* W4A16 weights (the W4A16 PR, sections "1. Packed fp16 dequant" and "2.
 * dtype-aware gfx1151 tile selection").  K % 128 == 0, group_size a power of
 * two >= 32, K % group_size == 0; has_zp selects the asymmetric (stored
 * zero-points) or symmetric (zero-point 8) variant and must match the
 * packing. */
int qgemm_w4a16(const void *X, const void *Wpacked, void *Y, int64_t M, int64_t N, int64_t K, int64_t group_size,
                int has_zp, int dtype, void *stream);

/* ---- tile selection and forced rungs (tests and benchmarks) -------------
 * The M-ladder (the W4A16 PR, "2. dtype-aware gfx1151 tile selection": a
 * tile per M bucket and dtype, with a K block that never straddles a
 * quantization group) maps (format, M, N, K, dtype) to a rung.
 * qgemm_select_rung writes 8 integers:
 *   [0] rung id  [1] rows per tile  [2] columns per tile  [3] K per step
 *   [4] waves per workgroup  [5] K-split ways (inside a workgroup, times the
 *       K slices across workgroups for mfma32-64x64-sk)
 *   [6] output tiles along N  [7] output tiles along M
 * and returns QGEMM_OK, or an error for an illegal shape.  num_rungs and
 * rung_name (NULL for an unknown rung) name the rungs; rung_info fills the
 * same integers for a given rung. */
int qgemm_num_rungs(void);
const char *qgemm_rung_name(int rung);
int qgemm_select_rung(int format, int64_t M, int64_t N, int64_t K, int dtype, int32_t *info8);
int qgemm_rung_info(int rung, int format, int64_t M, int64_t N, int64_t K, int dtype, int32_t *info8);

/* Workspace of the rungs that split K across workgroups (mfma32-64x64-sk and
 * mfma32-768x64-sk: the batched-prefill post's K-parallel row reduction, "The
 * fix: K-parallel batched DMMV", carried across workgroups with one
 * reduction at the end):
 * the bytes a qgemm_gemm_rung (layout QGEMM_X_ROW) or qgemm_gemm_xf
 * (QGEMM_X_FRAG) call with these arguments needs, S*M*N*4 rounded so that
 * each of the S <= 8 slices of fp32 partial sums starts 16-byte aligned; 0
 * when the rung (rung = -1: the ladder's choice for that layout) needs none,
 * for M = 0, or for illegal arguments.  For W4A16 the group size does not
 * change the answer. */
size_t qgemm_workspace_bytes(int format, int rung, int layout, int64_t M, int64_t N, int64_t K, int dtype);

/* The format entry points with the rung forced (rung = -1 selects as
 * qgemm_q4k/q6k/w4a16 do; the W4A16 PR, "2. dtype-aware gfx1151 tile
 * selection").  group_size/has_zp are ignored for k-quants.
 * mfma32-64x64-sk splits K into S slices across workgroups (S = 1..8, as
 * many as keep the grid within two workgroups per CU and each of a slice's
 * four K groups at least four whole 128-wide chunks), each writing fp32
 * partial sums of its 64x64 tiles to `workspace` (device, 16-byte aligned,
 * caller-owned, at least qgemm_workspace_bytes); a second launch adds the S
 * slices in slice order and rounds once into Y, so Y is deterministic, but
 * its fp32 summation order differs from the other rungs'.  mfma32-768x64-sk
 * does the same with 768x64 tiles (S = 1..8, as many as keep the grid within
 * one round of the 256 CUs and each slice at least two chunks).  Such a call
 * with workspace_bytes below that size (NULL included) returns
 * QGEMM_ERR_SIZE before any launch; the other rungs ignore both workspace
 * arguments. */
int qgemm_gemm_rung(int format, int rung, const void *X, const void *Wpacked, void *Y, int64_t M, int64_t N,
                    int64_t K, int64_t group_size, int has_zp, int dtype, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ---- fragment-major activations ---------------------------------------------
 * A second layout of X, made for the MFMA kernels: 32-row blocks one after
 * the other, each a sequence of 128-wide K chunks; inside a chunk, eight
 * 16-wide k-steps of 512 elements, each two halves (k%16 < 8, then >= 8) of
 * 32 rows x 8 consecutive k.  Element X[m][k] sits at
 *     ((m/32 * K/128 + k/128) * 8 + (k/16)%8) * 512 + ((k/8)%2 * 32 + m%32) * 8 + k%8
 * and rows M .. 32*ceil(M/32)-1 of the last block hold zeros.  One
 * activation operand of a 32x32x16 MFMA (32 rows x 16 k) is then 1 KB of
 * contiguous memory instead of 32 separate 32-byte pieces of rows K apart:
 * the layout lesson of the delta-net page ("Gap #2: State Layout": one cache
 * line per read instead of 32).  The layout is this library's own; it
 * changes where X is read, not what is computed.
 *
 * qgemm_xf_bytes: bytes of the fragment-major copy of an M x K matrix
 *   (2 * K * 32*ceil(M/32)); 0 for M < 0, K not a positive multiple of 128,
 *   or sizes beyond int32.
 * qgemm_x_to_xf: writes that copy of the row-major X [M][K] (fp16 or bf16
 *   bits; the copy moves 16-bit elements and ignores the type) into Xf
 *   (device, 16-byte aligned, qgemm_xf_bytes(M, K) bytes, caller-owned, not
 *   overlapping X).  One launch on `stream`; M = 0 is a no-op.  Errors:
 *   QGEMM_ERR_SHAPE, _NULL, _ALIGN, _HIP.
 * qgemm_gemm_xf: qgemm_gemm_rung with X given in the fragment-major layout
 *   (M and K are the logical sizes), workspace as there.  For the same rung,
 *   Y is bit-identical to qgemm_gemm_rung's on the row-major X: the kernels
 *   and their accumulation order are the same, only the activation addresses
 *   differ.  rung = -1 selects from the ladder tuned for this layout
 *   (qgemm_select_rung_xf), which may pick mfma32-64x64-sk (33..64 rows over
 *   a long K) or mfma32-768x64-sk (513..768 rows of Q4_K or Q6_K over K >=
 *   12288, e.g. 658 x 12288 -> 4096 needs 43 MB): size the workspace with
 *   qgemm_workspace_bytes(..., QGEMM_X_FRAG, ...). */
size_t qgemm_xf_bytes(int64_t M, int64_t K);
int qgemm_x_to_xf(const void *X, void *Xf, int64_t M, int64_t K, void *stream);
int qgemm_gemm_xf(int format, int rung, const void *Xf, const void *Wpacked, void *Y, int64_t M, int64_t N,
                  int64_t K, int64_t group_size, int has_zp, int dtype, void *workspace, size_t workspace_bytes,
                  void *stream);
int qgemm_select_rung_xf(int format, int64_t M, int64_t N, int64_t K, int dtype, int32_t *info8);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * qgemm_gemm_xf without the workspace arguments.  A call whose rung splits K
 * across workgroups keeps its partial sums in a fixed device array of the
 * library, QGEMM_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the first
 * such call on a GPU until the process ends; a call that would need more
 * (qgemm_workspace_bytes with QGEMM_X_FRAG above that size) returns
 * QGEMM_ERR_SIZE before any launch and says so on stderr.  The library
 * allocates nothing in it.  Every call on one GPU shares that array: calls
 * that overlap on one GPU (two streams, two host threads) race, so order
 * them (e.g. one stream); a call leaves the array's contents behind and the
 * next one needs none of them.  Other arguments, results and errors as
 * qgemm_gemm_xf; Y is bit-identical to qgemm_gemm_xf's. */
#define QGEMM_NOALLOC_SCRATCH_BYTES (16 << 20)
int qgemm_gemm_xf_noalloc(int format, int rung, const void *Xf, const void *Wpacked, void *Y, int64_t M, int64_t N,
                          int64_t K, int64_t group_size, int has_zp, int dtype, void *stream);

/* ---- logical dequant --------------------------------------------------------
 * Writes the unpacked weights as logical Wout[K][N] (row-major, dtype
 * elements, device, caller-owned) with the same device unpack code the
 * GEMMs use (the sparkinfer PR, "Proof of speedup": the dequant is checked
 * bit for bit, with an FNV-1a digest, against the reference values).  The
 * fused GEMMs never call it; it exists to check the unpack bit for bit in
 * the plain W[K][N] order.  Errors as qgemm_w4a16 (group_size ignored for
 * the k-quants). */
int qgemm_dequant(int format, const void *Wpacked, void *Wout, int64_t N, int64_t K, int64_t group_size, int has_zp,
                  int dtype, void *stream);

/* Grouped per-expert GEMM (the batched-prefill post, "What this did not
 * solve": a batched per-expert matmul that amortizes each expert's weights
 * over its routed tokens; the routing itself is not part of it).  X [T][K]
 * holds the routed token rows grouped by expert: rows offsets[e] ..
 * offsets[e+1]-1 use expert e, whose packed weights (the layout of the
 * format's packer, N x K) start at Wpacked + e * (packed bytes of one
 * expert), so Wpacked holds E times the packed bytes; Y [T][N] receives
 * their products in the same rows.  `offsets` (E+1 int32, 4-byte aligned)
 * is DEVICE memory, read by the kernel, so the caller needs no host copy of
 * the counts; it must be non-decreasing with offsets[0] = 0 and offsets[E] =
 * T.  The kernel clamps every offset into [0, T] and to at least the
 * previous one, so any contents stay inside X, Y and W (bad offsets only
 * give wrong rows).  Rows outside [offsets[0], offsets[E]) are not written.
 * One launch on `stream`, planned from T, E, N and K alone (the counts
 * stay on the device): qgemm_grouped_plan below names the kernel.  Results
 * as qgemm_gemm_rung for each expert.  Errors as qgemm_w4a16 (group_size
 * ignored for the k-quants), plus QGEMM_ERR_SHAPE for E < 1 or a grid
 * beyond ceil(T/16) + E = 65535, QGEMM_ERR_ALIGN when one expert's packed
 * size is not a multiple of 16 bytes; T = 0 is a no-op.
 *
 * qgemm_grouped_xf: the same product with X given as the fragment-major copy
 * of the T routed rows (qgemm_x_to_xf of X [T][K]; Xf holds
 * qgemm_xf_bytes(T, K) bytes, device, 16-byte aligned, caller-owned), the
 * layout of qgemm_gemm_xf (the delta-net page, "Gap #2: State Layout": one
 * cache line per activation read instead of one per row).  An expert's rows
 * may start anywhere inside a 32-row block.  The plan is qgemm_grouped's and
 * Y is bit-identical to qgemm_grouped's.  Arguments, ownership and errors as
 * qgemm_grouped.
 *
 * qgemm_grouped_plan: the launch both grouped calls make for T routed rows,
 * E experts and an N x K weight matrix per expert, in 8 integers (host
 * memory, caller-owned):
 *   [0] kernel: 0 the direct kernel (16 or 32 rows by 64 columns per
 *       workgroup, K split over [4] waves when the grid is small), 1 the
 *       shared-activation kernel (four waves over 128 columns that read each
 *       chunk of their rows' activations once, through LDS)
 *   [1] rows per tile  [2] columns per tile  [3] waves per workgroup
 *   [4] K-split ways inside a workgroup  [5] grid x  [6] grid y (row-tile
 *       slots: an upper bound on the tiles of all experts)  [7] 0
 * The shared kernel serves more than 16 rows per expert on average
 * (ceil(T/E)) once the grid fills the chip without a K split, with 32-row
 * tiles up to 48 rows per expert and 80-row tiles above.  Returns
 * QGEMM_ERR_NULL for a NULL info8, QGEMM_ERR_SHAPE for T < 0, E < 1, N < 1,
 * K not a positive multiple of 128 or a grid beyond ceil(T/16) + E = 65535,
 * else QGEMM_OK. */
int qgemm_grouped(int format, const void *X, const void *Wpacked, void *Y, const int32_t *offsets, int64_t E, int64_t T,
                  int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream);
int qgemm_grouped_xf(int format, const void *Xf, const void *Wpacked, void *Y, const int32_t *offsets, int64_t E,
                     int64_t T, int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream);
int qgemm_grouped_plan(int64_t T, int64_t E, int64_t N, int64_t K, int32_t *info8);

/* The staged arm (the dequant-scratch post, "The two passes hiding inside
 * one matmul": unpack to a 16-bit scratch, then a GEMM that reads it), kept
 * beside the fused path to measure what fusing saves on this GPU.  Step one
 * unpacks every weight of Wpacked with the fused path's unpack into
 * `scratch` (device, 16-byte aligned, at least qgemm_staged_scratch_bytes(N,
 * K) bytes, caller-owned; 2 bytes per weight, N padded to whole panels of
 * 16, in the order the streaming kernel consumes: per (panel, 128-wide K
 * chunk) 4 KB laid out [word 0..3][run 16g+col][16 bytes], word i of run g
 * of column col holding k = 128c + 32g + 8i .. +7 of that column, two
 * weights per 32-bit word, the lower k in the low half).  Step two is the
 * 128x128 streaming kernel of the fused path with its unpack replaced by
 * loads of those words, so Y equals the fused `mfma32-128x128` rung's Y bit
 * for bit.  Both launches go on `stream`.  Arguments and errors as
 * qgemm_gemm_rung (group_size ignored for the k-quants), plus
 * QGEMM_ERR_SIZE when scratch_bytes is too small and QGEMM_ERR_NULL when
 * scratch is NULL.  M = 0 still fills the scratch.
 * qgemm_staged_scratch_bytes returns 0 for an illegal N or K. */
size_t qgemm_staged_scratch_bytes(int64_t N, int64_t K);
int qgemm_staged(int format, const void *X, const void *Wpacked, void *scratch, size_t scratch_bytes, void *Y, int64_t M,
                 int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype, void *stream);

/* ---- int8-activation variant ----------------------------------------------
 * The other operand of the same idea (the dequant-scratch post, "Where the
 * gap stands now": activation quantization and weight-dequant fusion keep
 * each operand compressed until the multiply; the sparkinfer PR, "Summary":
 * a single-pass row quantize feeding an int8-native prefill GEMM, weights
 * dequantized to int8 rows).  The pages fix neither the scale granularity
 * nor the rounding; this library's reading, every step defined to the bit:
 *   weights     w32 = RN_f32(exact weight of the unpack contract above);
 *               per output column n: amax_n = max_k |w32[k][n]|,
 *               r_n = RN_f32(127/amax_n), s_n = RN_f32(amax_n/127);
 *               code qw = RNE(w32 * r_n) (the product exact, |qw| <= 127)
 *   activations per row m the same on X (exact in binary32): r_m, s_m, qx
 *   output      Y[m][n] = RN_t( RN_f32( RN_f32(acc) * RN_f32(s_m * s_n) ) ),
 *               acc = sum_k qx*qw exactly (int32)
 * with r = s = 0 when amax < 2^-96 (only a bf16 row gets there).  The
 * weight codes are never stored: the GEMM unpacks the packed bytes and
 * requantizes them on the way into the int8 MFMA operand, so W stays at its
 * packed size in HBM.  This path is an approximation of X . dequant(W) by
 * construction (int8 codes); its contract is bit-exactness against the
 * definition above, not the fp16 path's error bound.
 *
 * qgemm_i8_colscale: the per-column factors of one packed weight (the same
 *   Wpacked, N, K, group_size, has_zp as the GEMMs), once at load: r_n into
 *   rw[N] and s_n into sw[N] (device floats, 4-byte aligned, caller-owned).
 *   One launch on `stream`.  Errors as qgemm_dequant, without a dtype.
 * qgemm_i8_xq_bytes: bytes of the int8 activation copy, 32*ceil(M/32)*K; 0
 *   for M < 0, K not a positive multiple of 32, or sizes beyond int32.
 * qgemm_i8_quantize: X [M][K] row-major (dtype bits, device, 16-byte
 *   aligned) -> codes Xq (device, 16-byte aligned, qgemm_i8_xq_bytes bytes)
 *   and s_m into sx[M] (device floats).  Xq is fragment-major: 32-row
 *   blocks, each a sequence of 32-wide k-steps of 1 KB in which lane
 *   (r, h) holds row r, k = 32s + 16h .. +15, i.e. code (m, k) at
 *       (m/32)*32*K + (k/32)*1024 + ((k/16)%2)*512 + (m%32)*16 + k%16,
 *   rows M .. 32*ceil(M/32)-1 zero: one 1 KB piece is one int8 MFMA
 *   operand.  X must be finite.  One launch (one wave per row, four rows per
 *   workgroup, each row read once); M = 0 is a no-op.  Errors:
 *   QGEMM_ERR_SHAPE, _DTYPE, _NULL, _ALIGN, _HIP.
 * qgemm_i8_gemm: Y [M][N] (dtype, row-major, 16-byte aligned) from Xq and sx
 *   of qgemm_i8_quantize and Wpacked with rw and sw of qgemm_i8_colscale.
 *   rung -1 picks from this path's own ladder (qgemm_i8_select_rung), else
 *   0 .. qgemm_i8_num_rungs()-1; every rung gives the same bits.  K at most
 *   131072 (int32 sums stay exact).  One launch on `stream` (two for
 *   i8-64x64-sk, which splits K into up to 8 slices across workgroups,
 *   writes each slice's int32 partial sums to `workspace` (device, 16-byte
 *   aligned, caller-owned, at least qgemm_i8_workspace_bytes) and adds them,
 *   exactly, in the epilogue launch; with a smaller workspace, NULL
 *   included, it returns QGEMM_ERR_SIZE before any launch); M = 0 is a
 *   no-op.  Errors as qgemm_gemm_rung.
 * qgemm_i8_workspace_bytes: the workspace such a call needs (rung -1: the
 *   int8 ladder's choice), 0 when it needs none or the arguments are
 *   illegal. */
size_t qgemm_i8_xq_bytes(int64_t M, int64_t K);
int qgemm_i8_quantize(const void *X, void *Xq, float *sx, int64_t M, int64_t K, int dtype, void *stream);
int qgemm_i8_colscale(int format, const void *Wpacked, float *rw, float *sw, int64_t N, int64_t K, int64_t group_size,
                      int has_zp, void *stream);
int qgemm_i8_gemm(int format, int rung, const void *Xq, const float *sx, const void *Wpacked, const float *rw,
                  const float *sw, void *Y, int64_t M, int64_t N, int64_t K, int64_t group_size, int has_zp, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream);
size_t qgemm_i8_workspace_bytes(int format, int rung, int64_t M, int64_t N, int64_t K);

/* The int8 ladder (the W4A16 PR, "2. dtype-aware gfx1151 tile selection",
 * applied to this path's own tiles): rung count and names (as
 * qgemm_num_rungs / qgemm_rung_name); rung_info / select_rung fill info8 as
 * qgemm_rung_info (dtype does not enter: every rung computes the same
 * bits). */
int qgemm_i8_num_rungs(void);
const char *qgemm_i8_rung_name(int rung);
int qgemm_i8_rung_info(int rung, int format, int64_t M, int64_t N, int64_t K, int32_t *info8);
int qgemm_i8_select_rung(int format, int64_t M, int64_t N, int64_t K, int32_t *info8);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
