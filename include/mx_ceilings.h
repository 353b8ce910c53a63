/*
 * mx_ceilings.h -- C ABI of libmx_ceilings.so: the context kernels the
 * measurement of the hot path compares against.  They are not part of the
 * method and libmx.so does not use them.
 *
 *  - a device copy (16-byte non-temporal loads and stores): the HBM bandwidth
 *    a streaming kernel reaches on this GPU;
 *  - a read-mostly stream that writes one byte per four read, the byte mix
 *    of the bf16 -> MXFP4 quantizer (2 B in, 0.53 B out per element);
 *  - a loop of the block-scaled FP4 matrix instruction
 *    (V_MFMA_SCALE_F32_32X32X64_F8F6F4, E2M1 operands, E8M0 scales 2^0) fed
 *    by ds_read_b128 operand reads from LDS the way the tiled GEMM feeds it:
 *    8 waves per workgroup, one workgroup per CU, each wave 4 x 2 tiles of
 *    32 x 32, six 16-byte reads per eight instructions.  Its rate on random
 *    operand bytes is the matrix unit's sustained ceiling under the GPU's
 *    power limit (operands that toggle fewer bits run faster);
 *  - the tiled GEMM's operand stream alone: 32 KiB stages of 512 rows x 64
 *    bytes moved into LDS by buffer_load_dwordx4 ... lds, two stages in
 *    flight, a barrier per stage, 8 waves per workgroup, one workgroup per
 *    CU.  Its rate per CU bounds how fast a CU can be fed 256 x 256 tiles.
 *
 * Conventions: device pointers, 16-byte aligned; `stream` is a hipStream_t
 * passed as void*; work is enqueued and the call returns at once.  Return
 * value 0, 1 for a bad argument, 5 for a failed launch (the MX_* codes of
 * mx.h).
 */
#ifndef MX_CEILINGS_H
#define MX_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0, bytes) = src[0, bytes); bytes a multiple of 16. */
int mxc_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Reads src[0, bytes) and writes bytes/4 to dst: word i of dst is the xor of
 * the four words of 16-byte chunk i of src.  bytes a multiple of 16. */
int mxc_read4_write1(const void *src, void *dst, size_t bytes, void *stream);

/* Workgroups mxc_mfma_loop launches on the current device (one per CU). */
int mxc_mfma_loop_grid(void);

/* Floating-point operations of one mxc_mfma_loop call with this grid and
 * iteration count (2 * 32 * 32 * 64 per instruction, 16 instructions per
 * wave and iteration, 8 waves per workgroup). */
double mxc_mfma_loop_flops(int grid, int64_t iters);

/* The FP4 matrix-instruction loop: operands (32 KiB of device memory) are
 * copied to LDS once, then each wave multiplies fragments read from it for
 * `iters` iterations; out receives grid * 512 floats (each lane's sum of its
 * accumulators, so the work is not dead). */
int mxc_mfma_loop(const void *operands, float *out, int grid, int64_t iters, void *stream);

/* The LDS-DMA operand stream: `grid` workgroups each move `stages` stages of
 * 32 KiB (grid * stages * 32768 bytes in all) from src, a device buffer of
 * src_bytes (a multiple of 1 MiB: its 1 MiB windows are dealt to the
 * workgroups round robin); out receives grid * 512 words read back from LDS,
 * so the loads are not dead. */
int mxc_lds_dma(const void *src, size_t src_bytes, uint32_t *out, int grid, int stages, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MX_CEILINGS_H */
