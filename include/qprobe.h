/*
 * qprobe.h -- measurement aids for the benchmark (libqprobe.so), apart from
 * the GEMM library: the rate at which this GPU sustains dense MFMA work and
 * a plain streaming read, the two ceilings a fused-dequant GEMM is measured
 * against (the dequant-scratch post, "What the roofline says": a fused GEMM
 * sits on the compute roof, a weight stream on the bandwidth roof).
 */
#ifndef QPROBE_H
#define QPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QPROBE_OK 0
#define QPROBE_ERR_NULL (-1)
#define QPROBE_ERR_SHAPE (-2)
#define QPROBE_ERR_DTYPE (-3)
#define QPROBE_ERR_ALIGN (-4)
#define QPROBE_ERR_HIP (-7)
#define QPROBE_F16 0
#define QPROBE_BF16 1

/* Runs `blocks` workgroups of 256 threads, each wave issuing `iters` rounds
 * of four independent 32x32x16 MFMAs (fp16 or bf16 by `dtype`) on operands
 * read once from `operands` (device, 16-byte aligned, 32 KiB: 256 threads x
 * 8 vectors of 16 bytes), and writes one float per thread to `out` (device,
 * blocks*256 floats) so the work stays live.  FLOPs = 2*32*32*16 * 4 *
 * iters * 4 waves * blocks.  Timed on random operands it gives the MFMA rate
 * the chip sustains under its power limit.  Errors: QPROBE_ERR_NULL, _ALIGN,
 * _SHAPE (blocks or iters < 1), _DTYPE, _HIP. */
int qprobe_mfma(const void *operands, float *out, int blocks, int iters, int dtype, void *stream);

/* A plain streaming read of `bytes` (a positive multiple of 16) from `buf`
 * (device, 16-byte aligned) by `blocks` workgroups of 256 threads, 16-byte
 * loads at a grid stride, four in flight per thread; each thread writes one
 * 32-bit word to `out` (device, blocks*256 words) so the loads stay live.
 * Timed on buffers that miss the Infinity Cache it is the HBM read rate a
 * weight stream can hope for.  Errors: QPROBE_ERR_NULL, _ALIGN, _SHAPE,
 * _HIP. */
int qprobe_read(const void *buf, int64_t bytes, void *out, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QPROBE_H */
