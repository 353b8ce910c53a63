/*
 * mx_ref.h -- plain, slow CPU oracle for microscaling block quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library: every rule here is written
 * independently from the pages that define the method.
 *
 * Sources (cited by page title and section):
 *  - "Unveiling the Potential of Quantization with MXFP4: Strategies for
 *    Quantization Error Reduction" (Qiita walkthrough, Sec. 2 background: the
 *    MXFP4 / NVFP4 component lists; Sec. 3: QSNR eq. (1)-(2), the 12x range of
 *    E2M1, the 4.25 / 4.5 bits-per-element figures; Sec. 4: OAS and MBS).
 *  - "Is Finer Better? The Limits of Microscaling Formats in LLMs" (gist.science
 *    technical summary: UE4M3 smallest scale 2^-9, UE5M3 2^-17, per-tensor scale).
 *  - "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *    Quantization" (gist.science technical summary, Sec. 2.2: block-wise
 *    Hadamard rotation fused into activation quantization).
 *  - the ARITH 2025 MX-training report (fmread.com academic report, "research
 *    findings"): E2M1 / INT4 / E3M0 element types, RTNE / stochastic / ceil
 *    rounding, symmetric vs asymmetric scaling, row / column / 2D blocks.
 *  - The MX family also has 8-bit elements ("Unveiling the Potential of
 *    Quantization with MXFP4", current state, Sec. 1 and 6: MX formats of 8,
 *    6 and 4 bits; the proposed methods apply to MXFP8 and MXFP6).  The FP6
 *    and FP8 element encodings themselves (E2M3, E3M2, E4M3, E5M2) are the OCP
 *    MX definitions, which the pages build on but do not print.
 *
 * Every function takes host pointers.  Return codes: 0 ok, 1 bad argument,
 * 2 unsupported combination.
 */
#ifndef MX_REF_H
#define MX_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { REF_E2M1 = 0, REF_INT4 = 1, REF_FP6_E2M3 = 2, REF_FP6_E3M2 = 3, REF_E3M0 = 4,
       REF_FP8_E4M3 = 5, REF_FP8_E5M2 = 6 };
/* block-scale types */
enum { REF_SC_E8M0 = 0, REF_SC_UE4M3 = 1, REF_SC_NVFP4 = 2, REF_SC_UE5M3 = 3, REF_SC_E3M0 = 4 };
/* power-of-two exponent rule (E8M0 scales) */
enum { REF_RULE_FLOOR = 0, REF_RULE_CEIL = 1, REF_RULE_OAS = 2 };
/* element rounding */
enum { REF_RTNE = 0, REF_SR = 1, REF_CEIL = 2 };
/* tensor dtypes */
enum { REF_F32 = 0, REF_BF16 = 1 };

typedef struct {
    int32_t elem, scale, rule, round;
    int32_t block_rows, block_cols;
    int32_t asymmetric;
    int32_t hadamard;     /* 0 or the rotation size h */
    int32_t macro_cols;   /* 0 or 128 */
    float oas_tau;
    uint64_t seed, rng_offset;
} ref_format;

typedef struct {
    uint8_t *codes;        /* packed element codes, row-major            */
    uint8_t *scales;       /* one byte per block, row-major block grid   */
    uint16_t *offsets;     /* bf16 per block (asymmetric only)           */
    uint8_t *macro_scales; /* E4M3 byte per 1x128 macro block (MBS only) */
    float *tensor_scale;   /* NVFP4 fp32 per-tensor scale                */
    int32_t *ref_exp;      /* E3M0 reference exponent                    */
    int64_t rows, cols;
} ref_qtensor;

typedef struct {
    double sig2, err2;
    int64_t n, nonzero, flushed, zero_blocks;
} ref_stats;

int ref_quantize(const ref_format *f, int in_dtype, const void *x, int64_t rows,
                 int64_t cols, int64_t ld, ref_qtensor *out, void *dequant,
                 int dq_dtype, ref_stats *stats);
int ref_dequantize(const ref_format *f, const ref_qtensor *q, int out_dtype,
                   void *y, int64_t ld);
int ref_qsnr(int dtype, const void *ref, const void *approx, int64_t n,
             ref_stats *stats, double *qsnr_db);

/* scalar pieces, exported so the tests can pin them one by one */
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t ref_r16(uint64_t seed, uint64_t offset, uint64_t idx);
int ref_round_code(int elem, int asym, int mode, float v, uint32_t r16);
double ref_code_value(int elem, int asym, int code);
int ref_fp8_scale_code(int scale_kind, float t);
double ref_fp8_scale_value(int scale_kind, int code);
int ref_e8m0_exponent(int rule, float oas_tau, int elem, int asym, float amax);
float ref_hadamard_const(int h);
void ref_hadamard_row(int h, float *v);
void ref_set_threads(int n);
int ref_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
