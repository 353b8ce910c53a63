/*
 * mx.h -- C ABI of the MI355X (gfx950) microscaling block-quantization library
 * (libmx.so).
 *
 * The method.  A tensor is cut into small blocks; each block's largest
 * magnitude fixes one shared scale, every element is divided by it and rounded
 * onto a 4- or 6-bit grid, and codes and scales are stored packed.  Sources,
 * cited by page title and section:
 *   [U]  "Unveiling the Potential of Quantization with MXFP4: Strategies for
 *        Quantization Error Reduction" (walkthrough of the paper's Sec. 2-5):
 *        MXFP4 = 32 E2M1 elements + one E8M0 scale; NVFP4 = 16 E2M1 elements +
 *        one E4M3 scale + a per-tensor scale (Sec. 2, FP4 quantization);
 *        QSNR eq. (1) and (2), the 12x range of E2M1 and 4.25 / 4.5 bits per
 *        element (Sec. 3); Overflow-Aware Scaling and Macro Block Scaling, and
 *        the A.B^T product with block scales (Sec. 4, Fig. 5); the dot-product
 *        unit that resolves per-block scales and adds block partial sums
 *        (Sec. 3, Fig. 4).
 *   [F]  "Is Finer Better? The Limits of Microscaling Formats in LLMs"
 *        (technical summary): UE4M3 scales (smallest 2^-9) need a per-tensor
 *        scale on narrow tensors; UE5M3 (smallest 2^-17) does not.
 *   [B]  "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *        Quantization" (technical summary, Sec. 2.2): block-wise Hadamard
 *        rotation fused into activation quantization.
 *   [A]  ARITH 2025 report on MX quantization for LLM training (research flow
 *        step 3 and main results 3): element types E2M1 / INT4 / E3M0, RTNE,
 *        stochastic and ceil rounding, symmetric or asymmetric scaling, block
 *        size, row / column / 2D block organisation.
 *
 * Conventions for every entry point:
 *  - Every tensor pointer is a DEVICE pointer (memory of the current HIP
 *    device) unless the argument says "host".  The caller allocates and owns
 *    every buffer; the library allocates nothing and keeps no state between
 *    calls, so calls from several host threads on different streams are safe
 *    (the one exception, mx_quantize_noalloc, keeps a static scratch array
 *    per GPU; see there).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued and the call returns at once, except mx_qsnr, which waits.
 *  - Return value: MX_OK, or an MX_ERR_* code.  Every argument is checked
 *    before anything is launched; on error nothing is launched and no output
 *    is touched.  MX_ERR_HIP reports a failed launch.
 *  - 16-byte alignment is required of every tensor pointer (MX_ERR_ALIGN).
 */
#ifndef MX_H
#define MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MX_OK 0
#define MX_ERR_ARG 1          /* bad value, shape or null pointer            */
#define MX_ERR_UNSUPPORTED 2  /* valid format that this library does not run */
#define MX_ERR_ALIGN 3        /* pointer or leading dimension not aligned    */
#define MX_ERR_WORKSPACE 4    /* workspace missing or smaller than required  */
#define MX_ERR_HIP 5          /* a HIP launch failed                         */
#define MX_ERR_TOO_LARGE 6    /* mx_quantize_noalloc: the call needs more    *
                               * scratch than its static array holds         */

/* ---- element types [A], [U] --------------------------------------------
 * Codes are sign-magnitude unless noted; no format has Inf or NaN and every
 * element saturates at its largest magnitude.
 *  E2M1   4 bits, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, code = s<<3 | index
 *  INT4   4 bits; symmetric: -7..7 as a two's-complement nibble;
 *         asymmetric: 0..15 steps above the block offset
 *  FP6    6 bits, E2M3 (bias 1, max 7.5) or E3M2 (bias 3, max 28)
 *  E3M0   4 bits, magnitudes {0, 1/4, 1/2, 1, 2, 4, 8, 16} (exponent only)
 *  FP8    8 bits, E4M3 (bias 7, max 448) or E5M2 (bias 15, max 57344): the
 *         MX family's 8-bit elements ([U], current state: MX formats of 8, 6
 *         and 4 bits); their Inf/NaN codes are never produced               */
enum { MX_ELEM_E2M1 = 0, MX_ELEM_INT4 = 1, MX_ELEM_FP6_E2M3 = 2, MX_ELEM_FP6_E3M2 = 3,
       MX_ELEM_E3M0 = 4, MX_ELEM_FP8_E4M3 = 5, MX_ELEM_FP8_E5M2 = 6 };

/* ---- block-scale types [U], [F], [A] ------------------------------------
 *  E8M0   one byte, the power of two 2^(code-127); 0xFF marks a block that
 *         held a NaN or Inf
 *  UE4M3  unsigned E4M3 (bias 7, max 448, smallest 2^-9), RNE of amax/Qmax;
 *         0x7F marks a non-finite block
 *  NVFP4  UE4M3 block scale times an fp32 per-tensor scale g = amax_t/(Qmax*448)
 *  UE5M3  unsigned E5M3 (bias 15, smallest 2^-17, max 1.75*2^16), RNE of
 *         amax/Qmax, no per-tensor scale; 0xFF marks a non-finite block
 *  E3M0   three exponent bits read as a step-down c in 0..7 below a per-tensor
 *         exponent e_ref: scale = 2^(e_ref - c); 0xFF marks a non-finite block */
enum { MX_SCALE_E8M0 = 0, MX_SCALE_UE4M3 = 1, MX_SCALE_NVFP4 = 2, MX_SCALE_UE5M3 = 3,
       MX_SCALE_E3M0 = 4 };

/* ---- E8M0 exponent rule [U] Sec. 4 ---------------------------------------
 *  FLOOR  e = floor(log2 amax) - emax(element)        (the OCP MX rule)
 *  CEIL   smallest e with Qmax * 2^e >= amax           (amax maps onto Qmax)
 *  OAS    smallest e with tau * 2^e >= amax, Qmax <= tau < 2 Qmax: the block
 *         maximum may overflow Qmax (and saturate) so that fewer small values
 *         flush to zero.  E3M0 scales always use the CEIL rule.           */
enum { MX_RULE_FLOOR = 0, MX_RULE_CEIL = 1, MX_RULE_OAS = 2 };

/* ---- element rounding [A] ----------------------------------------------
 *  RTNE  nearest grid value, ties to the even code
 *  SR    stochastic: between neighbours lo <= |v| < hi go up iff r < f * 2^16,
 *        f = (|v| - lo) / (hi - lo), r = 16 bits of Philox4x32-10 with counter
 *        (idx/8, rng_offset), key seed, word (idx/2)%4, half idx%2, where idx =
 *        row*cols + col of the element in the tensor
 *  CEIL  the smallest grid value >= v (a negative value's magnitude rounds down) */
enum { MX_ROUND_RTNE = 0, MX_ROUND_SR = 1, MX_ROUND_CEIL = 2 };

enum { MX_DTYPE_F32 = 0, MX_DTYPE_BF16 = 1 };

/* A quantization format.  Block shapes: 1 x b (row), b x 1 (column) or b x b
 * (2D).  asymmetric: INT4 min/max scaling or E2M1 with a mid-range offset
 * (E8M0 scales only).  hadamard: 0, or h in {16, 32, 64, 128}: every
 * contiguous run of h values in a row is rotated by H_h / sqrt(h) before it is
 * quantized ([B]); codes, dequantized values and statistics are then in the
 * rotated domain.  macro_cols: 0, or 128 for Macro Block Scaling ([U] Sec. 4):
 * each 1x128 macro block gets a UE4M3 scale s_M in [1, 2] (the mantissa of
 * amax/Qmax), elements are divided by s_M, and 1 x block_cols sub-blocks get
 * E8M0 scales.  oas_tau: the OAS threshold.  seed, rng_offset: the SR key. */
typedef struct mx_format {
    int32_t elem, scale, rule, round;
    int32_t block_rows, block_cols;
    int32_t asymmetric;
    int32_t hadamard;
    int32_t macro_cols;
    float oas_tau;
    uint64_t seed, rng_offset;
} mx_format;

/* A quantized tensor (the struct is host memory; its pointers are device
 * memory; unused pointers may be NULL).  Layout, all row-major:
 *  codes         rows x (cols/2) bytes for 4-bit elements, element 2i in the
 *                low nibble of byte i; rows x (3*cols/4) bytes for FP6, a
 *                least-significant-bit-first stream of 6-bit codes per row;
 *                rows x cols bytes for FP8, one code per byte
 *  scales        (rows/block_rows) x (cols/block_cols) bytes
 *  offsets       same grid, bf16 (asymmetric only)
 *  macro_scales  rows x (cols/128) bytes of UE4M3 (Macro Block Scaling only)
 *  tensor_scale  one fp32 (NVFP4 only)
 *  ref_exp       one int32 (E3M0 scales only)                              */
typedef struct mx_qtensor {
    void *codes;
    void *scales;
    void *offsets;
    void *macro_scales;
    float *tensor_scale;
    int32_t *ref_exp;
    int64_t rows, cols;
} mx_qtensor;

/* Fidelity statistics [U] Sec. 3: sig2 = sum x^2 and err2 = sum (x - xq)^2
 * (float64), n elements, nonzero = #{x != 0}, flushed = #{x != 0 and xq = 0},
 * zero_blocks = #{blocks whose dequantized values are all zero}.
 * QSNR eq. (1) = 10 log10(sig2 / err2); MSE = err2 / n.                     */
typedef struct mx_stats {
    double sig2, err2;
    int64_t n, nonzero, flushed, zero_blocks;
} mx_stats;

/* Byte sizes of every output of mx_quantize for this format and shape, and of
 * the device workspace it needs (zero when it needs none).  `out` is host.
 * The storage is the format's bit budget: codes at the element width plus one
 * scale byte per block, 4 + 8/32 = 4.25 bits per element for 1 x 32 blocks
 * and 4.5 for 1 x 16 ([U] Sec. 3); plus the bf16 offsets, the macro scales
 * (one byte per 1 x 128), the fp32 tensor scale or the int32 reference
 * exponent where the format has them.  Returns MX_ERR_ARG / MX_ERR_UNSUPPORTED
 * for a format or shape mx_quantize would reject; `out` is then untouched.  */
typedef struct mx_sizes {
    size_t codes, scales, offsets, macro_scales, tensor_scale, ref_exp, workspace;
} mx_sizes;

int mx_query_sizes(const mx_format *f, int64_t rows, int64_t cols, mx_sizes *out);

/* Quantize x (rows x cols, row stride ld elements, dtype in_dtype) into `out`.
 * dequant (nullable): the dequantized tensor, rows x cols dense, dtype dq_dtype
 * (fake quantization).  stats (nullable, device): the statistics of x against
 * its dequantized values, written when the stream reaches them.  workspace:
 * device scratch of at least mx_query_sizes().workspace bytes (no initial
 * contents needed); calls that share one workspace must not overlap.
 * Shapes this library runs: rows % block_rows == 0 and cols % block_cols == 0;
 * row blocks b in {8, 16, 32, 64, 128, 256} with cols % 8 == 0; column and 2D
 * blocks b in {8, 16, 32}; ld a multiple of 16 bytes.                       */
int mx_quantize(const mx_format *f, int in_dtype, const void *x, int64_t rows,
                int64_t cols, int64_t ld, const mx_qtensor *out, void *dequant,
                int dq_dtype, mx_stats *stats, void *workspace, size_t ws_bytes,
                void *stream);

/* mx_quantize without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It runs the same kernels as mx_quantize;
 * what they need beyond the caller's inputs and outputs (the statistics
 * partials and the NVFP4 / E3M0 pre-pass maxima) goes into a static device
 * array of MX_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends.  The call itself allocates nothing (no hipMalloc,
 * no allocating library routine).  Its first call on a device looks up that
 * device's address of the array.
 *  - Limit: a call whose mx_query_sizes().workspace exceeds
 *    MX_NOALLOC_SCRATCH_BYTES returns MX_ERR_TOO_LARGE before any launch
 *    (4 MiB holds the statistics of about 350 M elements of row blocks).
 *    Calls that need no workspace (no statistics, no pre-pass) have no limit.
 *  - Every call on one GPU shares that GPU's array: calls that overlap in
 *    time on one GPU (two streams, two host threads) race and give wrong
 *    statistics or tensor scales.  Serialise them.  No initial contents are
 *    needed: every call writes what it reads.
 * Other arguments, errors and outputs: as mx_quantize.                      */
#define MX_NOALLOC_SCRATCH_BYTES (4u << 20)
int mx_quantize_noalloc(const mx_format *f, int in_dtype, const void *x, int64_t rows,
                        int64_t cols, int64_t ld, const mx_qtensor *out, void *dequant,
                        int dq_dtype, mx_stats *stats, void *stream);

/* One tensor of an mx_quantize_many call: mx_quantize's arguments for it,
 * without a dequantized output.  The struct and `out` are host memory; x,
 * out's buffers, stats and workspace are device memory.  workspace: at least
 * mx_query_sizes(f, rows, cols).workspace bytes when the job has statistics
 * or the format a pre-pass (NULL and 0 otherwise). */
typedef struct mx_qjob {
    const void *x;
    int64_t rows, cols, ld;
    const mx_qtensor *out;
    mx_stats *stats;
    void *workspace;
    size_t ws_bytes;
} mx_qjob;

/* Quantize several tensors of one format and input dtype, such as both
 * operands of a layer's A.B^T ([U] Sec. 4, Fig. 5): job i's codes, scales and
 * statistics are those mx_quantize(f, in_dtype, jobs[i].x, jobs[i].rows, ...)
 * writes.  jobs: host array of `count` entries (count >= 0; jobs may be NULL
 * when count is 0).
 *  - Dense MXFP4-style row jobs share launches: E2M1 elements, E8M0 scales
 *    (any rule), round to nearest, symmetric, no rotation, no macro scales,
 *    1 x b blocks, ld == cols.  Up to eight such jobs run in one quantization launch,
 *    their workgroups split in proportion to their sizes, and the statistics
 *    of all of them in one finalize launch, where calling mx_quantize for
 *    each would launch two kernels per tensor.  Every other job runs as
 *    mx_quantize runs it, one after another.
 *  - Every job is checked before the first launch, as mx_quantize checks its
 *    arguments (first failing job's status); MX_ERR_ARG also when two jobs that
 *    need a workspace name overlapping workspace bytes.
 *  - Jobs must not write overlapping memory; the order in which they run is
 *    unspecified.  Calls that share a workspace must not overlap. */
int mx_quantize_many(const mx_format *f, int in_dtype, const mx_qjob *jobs, int count, void *stream);

/* Dequantize q into y (rows x cols, row stride ld elements, dtype out_dtype
 * MX_DTYPE_F32 or MX_DTYPE_BF16, rounded to nearest even): each element is its
 * code's value times its block's scale (plus the block's offset when
 * asymmetric, times the macro scale under MBS, times the tensor scale for
 * NVFP4), the value mx_quantize's dequant output and statistics use.  This is
 * the fake (simulated) quantization with which [A] (research flow step 1)
 * studies MX formats on hardware that does not run them.  A block whose scale
 * code is NaN dequantizes to NaN.  q's buffers as mx_quantize wrote them;
 * ld >= cols with ld * element size a multiple of 16 (MX_ERR_ALIGN).        */
int mx_dequantize(const mx_format *f, const mx_qtensor *q, int out_dtype, void *y,
                  int64_t ld, void *stream);

/* QSNR eq. (1)/(2) of [U] Sec. 3 between two tensors of n elements: `ref` is
 * the reference A (or the product A.B), `approx` its quantized counterpart.
 * host_stats (host, nullable) receives the statistics (zero_blocks = 0) and
 * qsnr_db (host) the QSNR in dB (+inf when the two are equal).  Waits for the
 * stream.  Returns MX_ERR_ARG if ||ref|| = 0.  workspace: device scratch of at
 * least mx_qsnr_workspace_size(n) bytes.                                   */
size_t mx_qsnr_workspace_size(int64_t n);
int mx_qsnr(int dtype, const void *ref, const void *approx, int64_t n,
            mx_stats *host_stats, double *qsnr_db, void *workspace, size_t ws_bytes,
            void *stream);

/* Block-scaled GEMM ([U] Sec. 3 Fig. 4, Sec. 4 Fig. 5): C = deq(A) . deq(B)^T
 * with A an M x K and B an N x K quantized tensor in row blocks along K; fp32
 * accumulation, C (M x N, row stride ldc elements) in bf16 (rounded to nearest
 * even) or fp32.  Formats, per operand:
 *  - E8M0 scales on 1 x 32 blocks (any rule) with E2M1 (MXFP4), FP6 E2M3 /
 *    E3M2 (MXFP6) or FP8 E4M3 / E5M2 (MXFP8) elements, chosen independently
 *    for A and B (the mixed 4-/6-bit products of [A], main results; MX also
 *    has 8-bit formats, [U] current state): the gfx950 block-scaled
 *    FP8/FP6/FP4 matrix instruction.  MXFP4 operands may carry macro-block
 *    scales (macro_cols 128, [U] Sec. 4 MBS and Fig. 5: each 128-wide K step's
 *    partial product is multiplied by the two rows' UE4M3 macro scales).
 *  - E2M1 elements under UE4M3, NVFP4 (UE4M3 + fp32 tensor scale), UE5M3 or
 *    E8M0 scales on 1 x b blocks, b a multiple of 8 (when the other operand
 *    is not of the kind above): the codes times their block scales are
 *    decoded exactly, to fp16 when both operands have UE4M3 scales and to
 *    bf16 otherwise, and the fp16 / bf16 matrix instruction multiplies.
 *    Macro-block scales over E8M0 sub-blocks of other widths (the 1 x 128
 *    macro over 1 x 16 blocks, [U] Sec. 4 MBS) take this route too, with E8M0
 *    block scales on both operands: each block's scale is 2^e times its macro
 *    block's UE4M3 scale (exact in fp32) and the decode applies it.
 * Anything else (INT4 / E3M0 elements, asymmetric, rotated, column or 2D
 * blocks, macro scales on FP6 / FP8 or against fp8 block scales):
 * MX_ERR_UNSUPPORTED.  Shapes: K % 32 == 0 and
 * whole blocks (MX_ERR_ARG otherwise); any M, N.  E8M0 products with K a
 * multiple of 128 run on LDS-staged kernels (MXFP4 x MXFP4 without macro
 * scales and K a multiple of 1024 on the most tuned one), other K on a
 * register-only kernel; the decoded formats with 1 x 16 or 1 x 32 blocks and
 * K a multiple of 128 on an LDS-staged kernel, the rest register-only.  A
 * block whose scale code is NaN (E8M0 0xFF, UE4M3 0x7F, UE5M3 0xFF) makes its
 * row of C (column, for B) NaN.  macro_scales must be set when
 * the format has macro_cols, tensor_scale for NVFP4 (MX_ERR_ARG).          */
int mx_gemm(const mx_format *fa, const mx_qtensor *a, const mx_format *fb,
            const mx_qtensor *b, void *c, int64_t ldc, int c_dtype, void *stream);

/* Text for a status code (static storage). */
const char *mx_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MX_H */
