/*
 * mx_ref.c -- plain, slow CPU oracle for microscaling block quantization.
 *
 * TEST INFRASTRUCTURE ONLY (see mx_ref.h).  Scalar C, one block at a time, in
 * the order the method states its steps.  Element and scale rounding are done
 * by searching explicit value tables in double precision (every table value is
 * a short dyadic number, so every comparison below is exact).  Arithmetic that
 * the method performs on fp32 values (scale ratios, divisions by non-power-of-
 * two scales, Hadamard butterflies) is written as fp32 C expressions; the file
 * must be compiled without FMA contraction and without fast-math so that every
 * such expression is one IEEE fp32 operation with round-to-nearest-even.
 * Statistics accumulate in double.
 *
 * OpenMP only splits the loop over independent rows of blocks; per-row partial
 * sums are combined in a fixed order, so results do not depend on the thread
 * count.
 */
#include "mx_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0;

void ref_set_threads(int n) { g_threads = n; }
int ref_get_threads(void) {
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* fp32 / bf16 bits                                                          */
/* ------------------------------------------------------------------------ */
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float bf16_to_float(uint16_t h) { return float_of((uint32_t)h << 16); }

/* nearest bf16, ties to even (NaN stays a quiet NaN) */
static uint16_t bf16_nearest(float f) {
    uint32_t u = bits_of(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* largest bf16 value that is <= f (f finite) */
static uint16_t bf16_down(float f) {
    uint32_t u = bits_of(f);
    uint16_t hi = (uint16_t)(u >> 16);
    if ((u & 0xffffu) == 0) return hi;            /* already a bf16 value   */
    if (u >> 31) return (uint16_t)(hi + 1);       /* negative: grow |f|     */
    return hi;                                    /* positive: truncate     */
}

static int is_finite_f(float f) { return (bits_of(f) & 0x7f800000u) != 0x7f800000u; }

/* floor(log2(a)) for a finite a > 0 */
static int flog2(float a) { return ilogb((double)a); }

/* smallest integer e with Q * 2^e >= a (a > 0, Q > 0): the definition, by search */
static int e_ceil(float a, double Q) {
    int e = ilogb((double)a) - ilogb(Q);
    while (ldexp(Q, e) < (double)a) e++;
    while (ldexp(Q, e - 1) >= (double)a) e--;
    return e;
}

/* fp32 product with an exact power of two, as one rounding: fl(v * 2^k) */
static float times_pow2(float v, int k) { return (float)((double)v * ldexp(1.0, k)); }

/* ------------------------------------------------------------------------ */
/* element grids (non-negative magnitudes, ascending by code index)          */
/* ------------------------------------------------------------------------ */
typedef struct { int n; double g[128]; double qmax; int emax; int bits; } grid_t;

static grid_t G_E2M1, G_E3M0, G_INT4, G_UINT4, G_E2M3, G_E3M2, G_E4M3, G_E5M2;
static int grids_ready = 0;

static void build_grids(void) {
    /* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; max 6, min 0.5 */
    static const double e2m1[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
    /* E3M0 element: 3 exponent bits (bias 3), exponent field 0 means zero */
    static const double e3m0[8] = {0, 0.25, 0.5, 1, 2, 4, 8, 16};
    int i;
    G_E2M1.n = 8; G_E2M1.qmax = 6; G_E2M1.emax = 2; G_E2M1.bits = 4;
    G_E3M0.n = 8; G_E3M0.qmax = 16; G_E3M0.emax = 4; G_E3M0.bits = 4;
    for (i = 0; i < 8; i++) { G_E2M1.g[i] = e2m1[i]; G_E3M0.g[i] = e3m0[i]; }
    /* INT4 symmetric: integers -7..7 (two's complement nibble) */
    G_INT4.n = 8; G_INT4.qmax = 7; G_INT4.emax = 2; G_INT4.bits = 4;
    for (i = 0; i < 8; i++) G_INT4.g[i] = i;
    /* INT4 asymmetric: integers 0..15 above the block minimum */
    G_UINT4.n = 16; G_UINT4.qmax = 15; G_UINT4.emax = 3; G_UINT4.bits = 4;
    for (i = 0; i < 16; i++) G_UINT4.g[i] = i;
    /* FP6 E2M3 (bias 1) and E3M2 (bias 3), no Inf/NaN */
    G_E2M3.n = 32; G_E2M3.emax = 2; G_E2M3.bits = 6;
    G_E3M2.n = 32; G_E3M2.emax = 4; G_E3M2.bits = 6;
    for (i = 0; i < 32; i++) {
        int e = i >> 3, m = i & 7;
        G_E2M3.g[i] = e == 0 ? m / 8.0 : (1.0 + m / 8.0) * ldexp(1.0, e - 1);
        e = i >> 2; m = i & 3;
        G_E3M2.g[i] = e == 0 ? m / 16.0 : (1.0 + m / 4.0) * ldexp(1.0, e - 3);
    }
    G_E2M3.qmax = G_E2M3.g[31];
    G_E3M2.qmax = G_E3M2.g[31];
    /* FP8 E4M3 (bias 7; magnitude code 0x7F is NaN, so the largest value is
     * 0x7E = 448) and E5M2 (bias 15; 0x7C is Inf and above are NaN, so the
     * largest value is 0x7B = 57344), the OCP 8-bit MX element types.  As MX
     * elements they saturate at their largest finite value. */
    G_E4M3.n = 127; G_E4M3.emax = 8; G_E4M3.bits = 8;
    for (i = 0; i < 127; i++) {
        int e = i >> 3, m = i & 7;
        G_E4M3.g[i] = e == 0 ? m / 8.0 * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    }
    G_E5M2.n = 124; G_E5M2.emax = 15; G_E5M2.bits = 8;
    for (i = 0; i < 124; i++) {
        int e = i >> 2, m = i & 3;
        G_E5M2.g[i] = e == 0 ? m / 4.0 * ldexp(1.0, -14) : (1.0 + m / 4.0) * ldexp(1.0, e - 15);
    }
    G_E4M3.qmax = G_E4M3.g[126];
    G_E5M2.qmax = G_E5M2.g[123];
    grids_ready = 1;
}

static const grid_t *grid_for(int elem, int asym) {
    if (!grids_ready) build_grids();
    switch (elem) {
    case REF_E2M1: return &G_E2M1;
    case REF_INT4: return asym ? &G_UINT4 : &G_INT4;
    case REF_FP6_E2M3: return &G_E2M3;
    case REF_FP6_E3M2: return &G_E3M2;
    case REF_E3M0: return &G_E3M0;
    case REF_FP8_E4M3: return &G_E4M3;
    case REF_FP8_E5M2: return &G_E5M2;
    }
    return 0;
}

/*
 * Round v onto the element grid.  RTNE: nearest magnitude, ties to the even
 * code.  SR: between neighbours lo <= |v| < hi, go up iff r16 < f * 2^16 with
 * f = (|v| - lo) / (hi - lo).  CEIL: the smallest grid value >= v (toward +inf
 * on the signed value; a negative value rounds its magnitude down).  All modes
 * saturate at the largest magnitude and keep the sign of v (so a negative value
 * that rounds to zero gives a negative-zero code in the float formats).
 */
int ref_round_code(int elem, int asym, int mode, float v, uint32_t r16) {
    const grid_t *G = grid_for(elem, asym);
    int neg = signbit(v) ? 1 : 0;
    double m = fabs((double)v);
    int i;
    if (elem == REF_INT4 && asym && neg) m = 0;   /* below the block minimum */
    if (m >= G->g[G->n - 1]) {
        i = G->n - 1;
    } else {
        int lo = 0;
        double a, b;
        while (G->g[lo + 1] <= m) lo++;
        a = G->g[lo];
        b = G->g[lo + 1];
        if (mode == REF_RTNE) {
            double twice = 2.0 * m, mid = a + b;
            if (twice < mid) i = lo;
            else if (twice > mid) i = lo + 1;
            else i = (lo % 2 == 0) ? lo : lo + 1;
        } else if (mode == REF_SR) {
            double f = (m - a) / (b - a);
            i = ((double)r16 < f * 65536.0) ? lo + 1 : lo;
        } else {
            if (neg && !(elem == REF_INT4 && asym)) i = lo;
            else i = (m == a) ? lo : lo + 1;
        }
    }
    if (elem == REF_INT4) {
        if (asym) return i;
        return (neg ? -i : i) & 0xf;
    }
    return (neg << (G->bits - 1)) | i;
}

double ref_code_value(int elem, int asym, int code) {
    const grid_t *G = grid_for(elem, asym);
    if (elem == REF_INT4) {
        if (asym) return (double)(code & 0xf);
        return (double)((code & 0x8) ? (code & 0xf) - 16 : (code & 0xf));
    }
    {
        int sbit = G->bits - 1, idx = code & ((1 << sbit) - 1);
        double mag;
        if (idx >= G->n) return NAN;      /* FP8 Inf / NaN codes: never produced */
        mag = G->g[idx];
        return ((code >> sbit) & 1) ? -mag : mag;
    }
}

/* ------------------------------------------------------------------------ */
/* 8-bit scale formats                                                       */
/* ------------------------------------------------------------------------ */
/* unsigned E4M3 (bias 7, 0x7F is NaN, max 448, smallest 2^-9) and
 * unsigned E5M3 (bias 15, 0xFF is NaN, smallest 2^-17) */
double ref_fp8_scale_value(int kind, int code) {
    int e, m;
    if (kind == REF_SC_UE5M3) {
        if (code >= 0xff) return NAN;
        e = code >> 3; m = code & 7;
        return e == 0 ? m * ldexp(1.0, -17) : (1.0 + m / 8.0) * ldexp(1.0, e - 15);
    }
    if (code >= 0x7f) return NAN;
    e = code >> 3; m = code & 7;
    return e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
}

static int fp8_max_code(int kind) { return kind == REF_SC_UE5M3 ? 0xfe : 0x7e; }

/* nearest representable scale to t >= 0, ties to the even code, saturating */
int ref_fp8_scale_code(int kind, float t) {
    int maxc = fp8_max_code(kind);
    double td = (double)t;
    int c = 0;
    if (!(td < ref_fp8_scale_value(kind, maxc))) return maxc;   /* also +inf */
    while (ref_fp8_scale_value(kind, c + 1) <= td) c++;
    {
        double a = ref_fp8_scale_value(kind, c), b = ref_fp8_scale_value(kind, c + 1);
        double twice = 2.0 * td, mid = a + b;
        if (twice < mid) return c;
        if (twice > mid) return c + 1;
        return (c % 2 == 0) ? c : c + 1;
    }
}

/* E8M0 exponent of a block whose largest magnitude is amax > 0, clamped to
 * [-127, 127].  FLOOR: floor(log2 amax) - emax_elem (the OCP rule).
 * CEIL: smallest e with Qmax * 2^e >= amax (the block maximum maps onto the
 * largest element).  OAS: smallest e with tau * 2^e >= amax, Qmax <= tau < 2 Qmax
 * (the block maximum may overflow Qmax by up to tau / Qmax and then saturates). */
int ref_e8m0_exponent(int rule, float tau, int elem, int asym, float amax) {
    const grid_t *G = grid_for(elem, asym);
    int e;
    if (!(amax > 0)) return -127;
    /* a range that overflowed (max - offset beyond FLT_MAX): the largest scale */
    if (!is_finite_f(amax)) return 127;
    if (rule == REF_RULE_FLOOR) e = flog2(amax) - G->emax;
    else if (rule == REF_RULE_CEIL) e = e_ceil(amax, G->qmax);
    else e = e_ceil(amax, (double)tau);
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------------ */
/* counter-based RNG: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11)       */
/* ------------------------------------------------------------------------ */
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    int round;
    for (round = 0; round < 10; round++) {
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16 random bits for logical element idx: counter (idx/8, offset), key seed,
 * word (idx/2) mod 4 of the output, low half for even idx, high half for odd */
uint32_t ref_r16(uint64_t seed, uint64_t offset, uint64_t idx) {
    uint64_t j = idx >> 3;
    uint32_t ctr[4], key[2], out[4];
    ctr[0] = (uint32_t)j; ctr[1] = (uint32_t)(j >> 32);
    ctr[2] = (uint32_t)offset; ctr[3] = (uint32_t)(offset >> 32);
    key[0] = (uint32_t)seed; key[1] = (uint32_t)(seed >> 32);
    ref_philox4x32_10(ctr, key, out);
    {
        uint32_t w = out[(idx >> 1) & 3];
        return (idx & 1) ? (w >> 16) : (w & 0xffffu);
    }
}

/* ------------------------------------------------------------------------ */
/* block Hadamard rotation                                                   */
/* ------------------------------------------------------------------------ */
float ref_hadamard_const(int h) { return (float)(1.0 / sqrt((double)h)); }

/* in place on one chunk of h values: Sylvester order, stage s pairs (i, i+2^s)
 * with bit s of i clear, (a, b) -> (a + b, a - b), then scale by 1/sqrt(h) */
void ref_hadamard_row(int h, float *v) {
    int span, i;
    float c = ref_hadamard_const(h);
    for (span = 1; span < h; span <<= 1) {
        for (i = 0; i < h; i++) {
            if (i & span) continue;
            {
                float a = v[i], b = v[i + span];
                v[i] = a + b;
                v[i + span] = a - b;
            }
        }
    }
    for (i = 0; i < h; i++) v[i] = v[i] * c;
}

/* ------------------------------------------------------------------------ */
/* validation and layout                                                     */
/* ------------------------------------------------------------------------ */
static int is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

static int check_format(const ref_format *f, int64_t rows, int64_t cols) {
    const grid_t *G;
    int br = f->block_rows, bc = f->block_cols;
    if (f->elem < 0 || f->elem > REF_FP8_E5M2) return 1;
    if (f->scale < 0 || f->scale > REF_SC_E3M0) return 1;
    if (f->rule < 0 || f->rule > REF_RULE_OAS) return 1;
    if (f->round < 0 || f->round > REF_CEIL) return 1;
    if (rows < 0 || cols < 0 || br < 1 || bc < 1) return 1;
    if (rows % br || cols % bc) return 1;
    G = grid_for(f->elem, f->asymmetric);
    if (G->bits == 6 ? (cols % 4) : (cols % 2)) return 1;
    if (f->asymmetric) {
        if (f->elem != REF_E2M1 && f->elem != REF_INT4) return 2;
        if (f->scale != REF_SC_E8M0 || f->hadamard || f->macro_cols) return 2;
    }
    if (f->rule == REF_RULE_OAS && f->scale == REF_SC_E8M0) {
        if (!(f->oas_tau >= G->qmax && f->oas_tau < 2 * G->qmax)) return 1;
    }
    if (f->hadamard) {
        if (!is_pow2(f->hadamard) || f->hadamard < 2 || f->hadamard > 256) return 1;
        if (br != 1 || cols % f->hadamard) return 2;
    }
    if (f->macro_cols) {
        if (f->macro_cols != 128) return 1;
        if (br != 1 || 128 % bc || cols % 128 || f->scale != REF_SC_E8M0) return 2;
    }
    return 0;
}

static int64_t code_row_bytes(int elem, int64_t cols) {
    if (elem == REF_FP8_E4M3 || elem == REF_FP8_E5M2) return cols;
    return (elem == REF_FP6_E2M3 || elem == REF_FP6_E3M2) ? cols * 3 / 4 : cols / 2;
}

/* element c of one row: 4-bit codes two per byte (even element in the low
 * nibble); 6-bit codes as a least-significant-bit-first stream; 8-bit codes
 * one per byte */
static void put_code(uint8_t *row, int bits, int64_t c, int code) {
    if (bits == 8) {
        row[c] = (uint8_t)code;
    } else if (bits == 4) {
        uint8_t *p = row + c / 2;
        if (c % 2 == 0) *p = (uint8_t)((*p & 0xf0) | code);
        else *p = (uint8_t)((*p & 0x0f) | (code << 4));
    } else {
        int64_t bit;
        int k;
        for (k = 0; k < 6; k++) {
            bit = 6 * c + k;
            if ((code >> k) & 1) row[bit / 8] |= (uint8_t)(1u << (bit % 8));
            else row[bit / 8] &= (uint8_t)~(1u << (bit % 8));
        }
    }
}

static int get_code(const uint8_t *row, int bits, int64_t c) {
    if (bits == 8) return row[c];
    if (bits == 4) return (c % 2 == 0) ? (row[c / 2] & 0xf) : (row[c / 2] >> 4);
    {
        int code = 0, k;
        for (k = 0; k < 6; k++) {
            int64_t bit = 6 * c + k;
            code |= ((row[bit / 8] >> (bit % 8)) & 1) << k;
        }
        return code;
    }
}

static float load_elem(int dtype, const void *x, int64_t i) {
    if (dtype == REF_BF16) return bf16_to_float(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

static void store_elem(int dtype, void *y, int64_t i, float v) {
    if (dtype == REF_BF16) ((uint16_t *)y)[i] = bf16_nearest(v);
    else ((float *)y)[i] = v;
}

/* ------------------------------------------------------------------------ */
/* quantization                                                              */
/* ------------------------------------------------------------------------ */
typedef struct {
    const ref_format *f;
    const grid_t *G;
    int64_t rows, cols, nbc;      /* nbc: blocks per block-row */
    const float *X;               /* working fp32 copy, rows x cols     */
    float g;                      /* NVFP4 per-tensor scale             */
    int e_ref;                    /* E3M0 reference exponent            */
    ref_qtensor *out;
    float *DQ;                    /* dequantized fp32, rows x cols      */
} qctx;

/* quantize the value v (already divided by its scale) for logical element idx */
static int round_elem(const qctx *q, float v, int64_t idx) {
    uint32_t r = 0;
    if (q->f->round == REF_SR) r = ref_r16(q->f->seed, q->f->rng_offset, (uint64_t)idx);
    return ref_round_code(q->f->elem, q->f->asymmetric, q->f->round, v, r);
}

static float elem_value(const qctx *q, int code) {
    return (float)ref_code_value(q->f->elem, q->f->asymmetric, code);
}

static int scale_nan_code(int kind) {
    if (kind == REF_SC_UE4M3 || kind == REF_SC_NVFP4) return 0x7f;
    return 0xff;
}

/* one block: rows [r0, r0+br), cols [c0, c0+bc) */
static void quantize_block(const qctx *q, int64_t bi, int64_t bj) {
    const ref_format *f = q->f;
    const grid_t *G = q->G;
    int br = f->block_rows, bc = f->block_cols, bits = G->bits;
    int64_t r0 = bi * br, c0 = bj * bc, r, c;
    int64_t rb = code_row_bytes(f->elem, q->cols);
    int64_t sidx = bi * q->nbc + bj;
    float amax = 0, mn = INFINITY, mx = -INFINITY;
    int finite = 1;

    for (r = r0; r < r0 + br; r++)
        for (c = c0; c < c0 + bc; c++) {
            float x = q->X[r * q->cols + c];
            if (!is_finite_f(x)) { finite = 0; continue; }
            if (fabsf(x) > amax) amax = fabsf(x);
            if (x < mn) mn = x;
            if (x > mx) mx = x;
        }

    if (!finite) {
        q->out->scales[sidx] = (uint8_t)scale_nan_code(f->scale);
        if (f->asymmetric) q->out->offsets[sidx] = 0;
        for (r = r0; r < r0 + br; r++)
            for (c = c0; c < c0 + bc; c++) {
                put_code(q->out->codes + r * rb, bits, c, 0);
                q->DQ[r * q->cols + c] = NAN;
            }
        return;
    }

    if (f->asymmetric && f->elem == REF_INT4) {
        /* min/max scaling: codes count steps of 2^e above the bf16 floor of the min */
        float mlo = bf16_to_float(bf16_down(mn));
        float R = mx - mlo;
        int e = (R > 0) ? ref_e8m0_exponent(f->rule, f->oas_tau, f->elem, 1, R) : -127;
        q->out->scales[sidx] = (uint8_t)(e + 127);
        q->out->offsets[sidx] = bf16_down(mn);
        for (r = r0; r < r0 + br; r++)
            for (c = c0; c < c0 + bc; c++) {
                float x = q->X[r * q->cols + c];
                float v = times_pow2(x - mlo, -e);
                int code = round_elem(q, v, r * q->cols + c);
                put_code(q->out->codes + r * rb, bits, c, code);
                q->DQ[r * q->cols + c] = mlo + times_pow2(elem_value(q, code), e);
            }
        return;
    }

    if (f->asymmetric) {
        /* E2M1 with a bf16 mid-range offset, then symmetric scaling of the rest.
         * The mid-range halves each end before adding (exact for normal values),
         * so it cannot overflow when both ends are near FLT_MAX. */
        uint16_t ob = bf16_nearest(mx * 0.5f + mn * 0.5f);
        float o = bf16_to_float(ob);
        float ymax = 0;
        int e;
        for (r = r0; r < r0 + br; r++)
            for (c = c0; c < c0 + bc; c++) {
                float y = q->X[r * q->cols + c] - o;
                if (fabsf(y) > ymax) ymax = fabsf(y);
            }
        e = ref_e8m0_exponent(f->rule, f->oas_tau, f->elem, 0, ymax);
        q->out->scales[sidx] = (uint8_t)(e + 127);
        q->out->offsets[sidx] = ob;
        for (r = r0; r < r0 + br; r++)
            for (c = c0; c < c0 + bc; c++) {
                float y = q->X[r * q->cols + c] - o;
                int code = round_elem(q, times_pow2(y, -e), r * q->cols + c);
                put_code(q->out->codes + r * rb, bits, c, code);
                q->DQ[r * q->cols + c] = times_pow2(elem_value(q, code), e) + o;
            }
        return;
    }

    if (f->scale == REF_SC_E8M0 || f->scale == REF_SC_E3M0) {
        int e, sc;
        if (f->scale == REF_SC_E8M0) {
            e = ref_e8m0_exponent(f->rule, f->oas_tau, f->elem, 0, amax);
            sc = e + 127;
        } else {
            /* three exponent bits, read as a step-down 0..7 below the tensor exponent */
            int cdown = 7;
            if (amax > 0) {
                cdown = q->e_ref - e_ceil(amax, G->qmax);
                if (cdown < 0) cdown = 0;
                if (cdown > 7) cdown = 7;
            }
            e = q->e_ref - cdown;
            sc = cdown;
        }
        q->out->scales[sidx] = (uint8_t)sc;
        for (r = r0; r < r0 + br; r++)
            for (c = c0; c < c0 + bc; c++) {
                float x = q->X[r * q->cols + c];
                int code = round_elem(q, times_pow2(x, -e), r * q->cols + c);
                put_code(q->out->codes + r * rb, bits, c, code);
                q->DQ[r * q->cols + c] = times_pow2(elem_value(q, code), e);
            }
        return;
    }

    {
        /* 8-bit floating scales: UE4M3, UE5M3, or UE4M3 times the tensor scale */
        int kind = f->scale == REF_SC_UE5M3 ? REF_SC_UE5M3 : REF_SC_UE4M3;
        float qmax = (float)G->qmax;
        float t = amax / qmax;
        float sb, S;
        int sc;
        if (f->scale == REF_SC_NVFP4) t = t / q->g;
        sc = ref_fp8_scale_code(kind, t);
        sb = (float)ref_fp8_scale_value(kind, sc);
        S = (f->scale == REF_SC_NVFP4) ? sb * q->g : sb;
        q->out->scales[sidx] = (uint8_t)sc;
        for (r = r0; r < r0 + br; r++)
            for (c = c0; c < c0 + bc; c++) {
                float x = q->X[r * q->cols + c];
                int code;
                float dq;
                if (S == 0) {
                    /* scale underflowed: every element of the block is a signed zero */
                    code = ref_round_code(f->elem, 0, REF_RTNE, signbit(x) ? -0.0f : 0.0f, 0);
                } else {
                    code = round_elem(q, x / S, r * q->cols + c);
                }
                dq = elem_value(q, code) * sb;
                if (f->scale == REF_SC_NVFP4) dq = dq * q->g;
                put_code(q->out->codes + r * rb, bits, c, code);
                q->DQ[r * q->cols + c] = dq;
            }
    }
}

/* macro-block scaling over one row: a UE4M3 value in [1, 2] per 1x128 macro
 * block (the mantissa of max|x| / Qmax), then E8M0 sub-blocks on x / s_M */
static void quantize_macro_row(const qctx *q, int64_t r, float *ybuf) {
    const ref_format *f = q->f;
    const grid_t *G = q->G;
    int bc = f->block_cols, bits = G->bits;
    int64_t rb = code_row_bytes(f->elem, q->cols);
    int64_t nmac = q->cols / 128, m, c, j;
    for (m = 0; m < nmac; m++) {
        const float *x = q->X + r * q->cols + m * 128;
        float M = 0, sM = 1.0f;
        int smc;
        for (c = 0; c < 128; c++)
            if (is_finite_f(x[c]) && fabsf(x[c]) > M) M = fabsf(x[c]);
        if (M > 0) {
            float t = M / (float)G->qmax;
            float mu = times_pow2(t, -flog2(t));      /* in [1, 2) */
            smc = ref_fp8_scale_code(REF_SC_UE4M3, mu);
            sM = (float)ref_fp8_scale_value(REF_SC_UE4M3, smc);
        } else {
            smc = ref_fp8_scale_code(REF_SC_UE4M3, 1.0f);
        }
        q->out->macro_scales[r * nmac + m] = (uint8_t)smc;
        for (c = 0; c < 128; c++) ybuf[c] = x[c] / sM;
        for (j = 0; j < 128 / bc; j++) {
            float amax = 0;
            int finite = 1, e;
            int64_t c0 = m * 128 + j * bc;
            int64_t sidx = r * q->nbc + c0 / bc;
            for (c = 0; c < bc; c++) {
                float y = ybuf[j * bc + c];
                if (!is_finite_f(y)) finite = 0;
                else if (fabsf(y) > amax) amax = fabsf(y);
            }
            if (!finite) {
                q->out->scales[sidx] = 0xff;
                for (c = 0; c < bc; c++) {
                    put_code(q->out->codes + r * rb, bits, c0 + c, 0);
                    q->DQ[r * q->cols + c0 + c] = NAN;
                }
                continue;
            }
            e = ref_e8m0_exponent(f->rule, f->oas_tau, f->elem, 0, amax);
            q->out->scales[sidx] = (uint8_t)(e + 127);
            for (c = 0; c < bc; c++) {
                float y = ybuf[j * bc + c];
                int code = round_elem(q, times_pow2(y, -e), r * q->cols + c0 + c);
                put_code(q->out->codes + r * rb, bits, c0 + c, code);
                q->DQ[r * q->cols + c0 + c] = times_pow2(elem_value(q, code), e) * sM;
            }
        }
    }
}

static float tensor_amax(const float *X, int64_t n) {
    float a = 0;
    int64_t i;
    for (i = 0; i < n; i++)
        if (is_finite_f(X[i]) && fabsf(X[i]) > a) a = fabsf(X[i]);
    return a;
}

int ref_quantize(const ref_format *f, int in_dtype, const void *x, int64_t rows,
                 int64_t cols, int64_t ld, ref_qtensor *out, void *dequant,
                 int dq_dtype, ref_stats *stats) {
    qctx q;
    float *X, *DQ;
    int64_t r, c, nbr, i;
    double *psig, *perr;
    int64_t *pnz, *pfl, *pzb;
    int rc = check_format(f, rows, cols);
    if (rc) return rc;
    if (ld < cols || !out || !out->codes || !out->scales) return 1;
    if (in_dtype != REF_F32 && in_dtype != REF_BF16) return 1;
    if (f->asymmetric && !out->offsets) return 1;
    if (f->macro_cols && !out->macro_scales) return 1;
    if (f->scale == REF_SC_NVFP4 && !out->tensor_scale) return 1;
    if (f->scale == REF_SC_E3M0 && !out->ref_exp) return 1;
    out->rows = rows;
    out->cols = cols;

    X = (float *)malloc(sizeof(float) * (size_t)(rows * cols + 1));
    DQ = (float *)malloc(sizeof(float) * (size_t)(rows * cols + 1));
    if (!X || !DQ) { free(X); free(DQ); return 1; }
    for (r = 0; r < rows; r++)
        for (c = 0; c < cols; c++) X[r * cols + c] = load_elem(in_dtype, x, r * ld + c);
    if (f->hadamard)
        for (r = 0; r < rows; r++)
            for (c = 0; c < cols; c += f->hadamard) ref_hadamard_row(f->hadamard, X + r * cols + c);

    q.f = f;
    q.G = grid_for(f->elem, f->asymmetric);
    q.rows = rows;
    q.cols = cols;
    q.nbc = cols / f->block_cols;
    q.X = X;
    q.g = 1.0f;
    q.e_ref = 0;
    q.out = out;
    q.DQ = DQ;
    if (f->scale == REF_SC_NVFP4) {
        /* per-tensor scale: map the tensor maximum onto Qmax * 448 */
        float at = tensor_amax(X, rows * cols);
        q.g = at > 0 ? at / ((float)q.G->qmax * 448.0f) : 1.0f;
        out->tensor_scale[0] = q.g;
    }
    if (f->scale == REF_SC_E3M0) {
        float at = tensor_amax(X, rows * cols);
        q.e_ref = at > 0 ? e_ceil(at, q.G->qmax) : 0;
        out->ref_exp[0] = q.e_ref;
    }

    nbr = rows / f->block_rows;
    if (f->macro_cols) {
#pragma omp parallel num_threads(ref_get_threads())
        {
            float ybuf[128];
            int64_t rr;
#pragma omp for schedule(static)
            for (rr = 0; rr < rows; rr++) quantize_macro_row(&q, rr, ybuf);
        }
    } else {
        int64_t bi;
#pragma omp parallel for schedule(static) num_threads(ref_get_threads())
        for (bi = 0; bi < nbr; bi++) {
            int64_t bj;
            for (bj = 0; bj < q.nbc; bj++) quantize_block(&q, bi, bj);
        }
    }

    if (dequant)
        for (r = 0; r < rows; r++)
            for (c = 0; c < cols; c++) store_elem(dq_dtype, dequant, r * cols + c, DQ[r * cols + c]);

    if (stats) {
        /* per block-row partial sums, combined in row order */
        psig = (double *)calloc((size_t)nbr + 1, sizeof(double));
        perr = (double *)calloc((size_t)nbr + 1, sizeof(double));
        pnz = (int64_t *)calloc((size_t)nbr + 1, sizeof(int64_t));
        pfl = (int64_t *)calloc((size_t)nbr + 1, sizeof(int64_t));
        pzb = (int64_t *)calloc((size_t)nbr + 1, sizeof(int64_t));
        {
            int64_t bi;
#pragma omp parallel for schedule(static) num_threads(ref_get_threads())
            for (bi = 0; bi < nbr; bi++) {
                int64_t rr, cc, bj;
                int br = f->block_rows, bc = f->block_cols;
                for (rr = bi * br; rr < (bi + 1) * br; rr++)
                    for (cc = 0; cc < cols; cc++) {
                        double xv = X[rr * cols + cc], dv = DQ[rr * cols + cc];
                        psig[bi] += xv * xv;
                        perr[bi] += (xv - dv) * (xv - dv);
                        if (xv != 0) {
                            pnz[bi]++;
                            if (dv == 0) pfl[bi]++;
                        }
                    }
                for (bj = 0; bj < q.nbc; bj++) {
                    int all_zero = 1;
                    for (rr = bi * br; rr < (bi + 1) * br && all_zero; rr++)
                        for (cc = bj * bc; cc < (bj + 1) * bc; cc++)
                            if (DQ[rr * cols + cc] != 0) { all_zero = 0; break; }
                    pzb[bi] += all_zero;
                }
            }
        }
        memset(stats, 0, sizeof(*stats));
        stats->n = rows * cols;
        for (i = 0; i < nbr; i++) {
            stats->sig2 += psig[i];
            stats->err2 += perr[i];
            stats->nonzero += pnz[i];
            stats->flushed += pfl[i];
            stats->zero_blocks += pzb[i];
        }
        free(psig); free(perr); free(pnz); free(pfl); free(pzb);
    }
    free(X);
    free(DQ);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* dequantization from the stored codes and scales                           */
/* ------------------------------------------------------------------------ */
int ref_dequantize(const ref_format *f, const ref_qtensor *qt, int out_dtype, void *y, int64_t ld) {
    const grid_t *G;
    int64_t rows, cols, rb, nbc, r, c;
    int br, bc, bits;
    int rc;
    if (!qt) return 1;
    rows = qt->rows;
    cols = qt->cols;
    rc = check_format(f, rows, cols);
    if (rc) return rc;
    if (ld < cols || !y) return 1;
    G = grid_for(f->elem, f->asymmetric);
    bits = G->bits;
    br = f->block_rows;
    bc = f->block_cols;
    rb = code_row_bytes(f->elem, cols);
    nbc = cols / bc;
#pragma omp parallel for schedule(static) private(c) num_threads(ref_get_threads())
    for (r = 0; r < rows; r++) {
        for (c = 0; c < cols; c++) {
            int64_t sidx = (r / br) * nbc + c / bc;
            int sc = qt->scales[sidx];
            int code = get_code(qt->codes + r * rb, bits, c);
            float val = (float)ref_code_value(f->elem, f->asymmetric, code);
            float out;
            if (sc == scale_nan_code(f->scale) && f->scale != REF_SC_E3M0) {
                out = NAN;
            } else if (f->scale == REF_SC_E3M0 && sc == 0xff) {
                out = NAN;
            } else if (f->asymmetric && f->elem == REF_INT4) {
                out = bf16_to_float(qt->offsets[sidx]) + times_pow2(val, sc - 127);
            } else if (f->asymmetric) {
                out = times_pow2(val, sc - 127) + bf16_to_float(qt->offsets[sidx]);
            } else if (f->macro_cols) {
                float sM = (float)ref_fp8_scale_value(REF_SC_UE4M3, qt->macro_scales[r * (cols / 128) + c / 128]);
                out = times_pow2(val, sc - 127) * sM;
            } else if (f->scale == REF_SC_E8M0) {
                out = times_pow2(val, sc - 127);
            } else if (f->scale == REF_SC_E3M0) {
                out = times_pow2(val, qt->ref_exp[0] - sc);
            } else {
                int kind = f->scale == REF_SC_UE5M3 ? REF_SC_UE5M3 : REF_SC_UE4M3;
                float sb = (float)ref_fp8_scale_value(kind, sc);
                out = val * sb;
                if (f->scale == REF_SC_NVFP4) out = out * qt->tensor_scale[0];
            }
            store_elem(out_dtype, y, r * ld + c, out);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* QSNR between two tensors: 10 log10( ||ref||^2 / ||ref - approx||^2 )       */
/* ------------------------------------------------------------------------ */
int ref_qsnr(int dtype, const void *ref, const void *approx, int64_t n, ref_stats *st, double *qsnr_db) {
    ref_stats s;
    int64_t i;
    if (n <= 0 || !ref || !approx) return 1;
    memset(&s, 0, sizeof(s));
    s.n = n;
    for (i = 0; i < n; i++) {
        double a = load_elem(dtype, ref, i), b = load_elem(dtype, approx, i);
        s.sig2 += a * a;
        s.err2 += (a - b) * (a - b);
        if (a != 0) {
            s.nonzero++;
            if (b == 0) s.flushed++;
        }
    }
    if (st) *st = s;
    if (!(s.sig2 > 0)) return 1;
    if (qsnr_db) *qsnr_db = s.err2 > 0 ? 10.0 * log10(s.sig2 / s.err2) : INFINITY;
    return 0;
}
