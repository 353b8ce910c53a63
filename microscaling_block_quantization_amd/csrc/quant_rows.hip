// quant_rows.hip -- quantization of 1 x b row blocks on gfx950 (all element
// types, scale types, rounding modes, asymmetric scaling, fused block
// Hadamard rotation and macro-block scaling), with optional fused dequantize
// and fidelity statistics.
//
// Work split: one thread owns CH consecutive elements of one row (16-byte
// loads); a block of b >= CH elements spans b/CH neighbouring lanes, which
// combine their maxima with cross-lane shuffles; b < CH puts CH/b blocks in a
// thread.  A Hadamard chunk of h elements spans h/CH lanes: butterflies with
// span < CH run in registers, the rest across lanes, in the same stage order
// as the definition ("Bridging the Gap ... Microscaling FP4 Quantization",
// Sec. 2.2, block-wise rotation fused into activation quantization).
// Macro Block Scaling ("Unveiling the Potential of Quantization with MXFP4",
// Sec. 4) spans 128/CH lanes.
#include <string.h>

#include "mx_kernels.hpp"

namespace mxk {
using namespace mxd;

namespace {

__device__ __forceinline__ float had_const(int h) {
    switch (h) {
    case 16: return 0.25f;
    case 32: return __uint_as_float(0x3E3504F3u);   // nearest fp32 to 1/sqrt(32)
    case 64: return 0.125f;
    default: return __uint_as_float(0x3DB504F3u);   // nearest fp32 to 1/sqrt(128)
    }
}

template <bool BF, int CH>
__device__ __forceinline__ void load_chunk(const QParams& p, int64_t r, int64_t c0, bool active,
                                           float (&x)[CH]) {
    if (!active) {
#pragma unroll
        for (int i = 0; i < CH; i++) x[i] = 0.f;
        return;
    }
    if constexpr (BF) {
        const uint16_t* src = static_cast<const uint16_t*>(p.x) + r * p.ld + c0;
#pragma unroll
        for (int v = 0; v < CH / 8; v++) {
            u32x4 w = ld_stream16(src + 8 * v);
            x[8 * v + 0] = bf16lo(w.x); x[8 * v + 1] = bf16hi(w.x);
            x[8 * v + 2] = bf16lo(w.y); x[8 * v + 3] = bf16hi(w.y);
            x[8 * v + 4] = bf16lo(w.z); x[8 * v + 5] = bf16hi(w.z);
            x[8 * v + 6] = bf16lo(w.w); x[8 * v + 7] = bf16hi(w.w);
        }
    } else {
        const float* src = static_cast<const float*>(p.x) + r * p.ld + c0;
#pragma unroll
        for (int v = 0; v < CH / 4; v++) {
            u32x4 w = ld_stream16(src + 4 * v);
            x[4 * v + 0] = __uint_as_float(w.x); x[4 * v + 1] = __uint_as_float(w.y);
            x[4 * v + 2] = __uint_as_float(w.z); x[4 * v + 3] = __uint_as_float(w.w);
        }
    }
}

// butterflies of H_h / sqrt(h) over the h-chunk this thread's CH values belong to
template <int CH>
__device__ __forceinline__ void hadamard(float (&x)[CH], int h) {
#pragma unroll
    for (int span = 1; span < CH; span <<= 1) {
#pragma unroll
        for (int i = 0; i < CH; i++) {
            if (i & span) continue;
            float a = x[i], b = x[i + span];
            x[i] = a + b;
            x[i + span] = a - b;
        }
    }
    for (int ls = 1; ls < h / CH; ls <<= 1) {
        const bool upper = (threadIdx.x & ls) != 0;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            float o = __shfl_xor(x[i], ls, 64);
            x[i] = upper ? (o - x[i]) : (x[i] + o);
        }
    }
    const float c = had_const(h);
#pragma unroll
    for (int i = 0; i < CH; i++) x[i] = x[i] * c;
}

__device__ __forceinline__ void store_codes(uint8_t* row, int bits, int64_t c0, const int* code, int n) {
    if (bits == 8) {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; i++)
            if (i < n) w[i >> 2] |= (uint32_t)(code[i] & 0xff) << (8 * (i & 3));
        if (n == 16) *reinterpret_cast<uint4*>(row + c0) = make_uint4(w[0], w[1], w[2], w[3]);
        else *reinterpret_cast<uint2*>(row + c0) = make_uint2(w[0], w[1]);
    } else if (bits == 4) {
        if (n == 16) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) lo |= (uint32_t)code[i] << (4 * i);
#pragma unroll
            for (int i = 0; i < 8; i++) hi |= (uint32_t)code[8 + i] << (4 * i);
            *reinterpret_cast<uint2*>(row + c0 / 2) = make_uint2(lo, hi);
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) w |= (uint32_t)code[i] << (4 * i);
            *reinterpret_cast<uint32_t*>(row + c0 / 2) = w;
        }
    } else {
        // 6-bit codes, least-significant bit first: 4 codes per 3 bytes
        uint32_t w[3] = {0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if (i >= n) break;
            int bit = 6 * i;
            w[bit >> 5] |= (uint32_t)code[i] << (bit & 31);
            if ((bit & 31) > 26) w[(bit >> 5) + 1] |= (uint32_t)code[i] >> (32 - (bit & 31));
        }
        uint8_t* dst = row + c0 * 3 / 4;
        if (n == 16) {
            uint32_t* d = reinterpret_cast<uint32_t*>(dst);
            d[0] = w[0]; d[1] = w[1]; d[2] = w[2];
        } else {
            uint16_t* d = reinterpret_cast<uint16_t*>(dst);
            d[0] = (uint16_t)w[0]; d[1] = (uint16_t)(w[0] >> 16); d[2] = (uint16_t)w[1];
        }
    }
}

template <int CH>
__device__ __forceinline__ void store_dq(const QParams& p, int64_t r, int64_t c0, const float (&d)[CH]) {
    if (p.dq_bf16) {
        uint16_t* dst = static_cast<uint16_t*>(p.dq) + r * p.cols + c0;
#pragma unroll
        for (int v = 0; v < CH / 8; v++) {
            uint4 w;
            w.x = bf16_rne(d[8 * v + 0]) | ((uint32_t)bf16_rne(d[8 * v + 1]) << 16);
            w.y = bf16_rne(d[8 * v + 2]) | ((uint32_t)bf16_rne(d[8 * v + 3]) << 16);
            w.z = bf16_rne(d[8 * v + 4]) | ((uint32_t)bf16_rne(d[8 * v + 5]) << 16);
            w.w = bf16_rne(d[8 * v + 6]) | ((uint32_t)bf16_rne(d[8 * v + 7]) << 16);
            reinterpret_cast<uint4*>(dst)[v] = w;
        }
    } else {
        float* dst = static_cast<float*>(p.dq) + r * p.cols + c0;
#pragma unroll
        for (int v = 0; v < CH / 4; v++)
            reinterpret_cast<float4*>(dst)[v] = make_float4(d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3]);
    }
}

__device__ __forceinline__ int nan_scale_code(int scale) {
    return (scale == SC_UE4M3 || scale == SC_NVFP4) ? 0x7f : 0xff;
}

template <int NTH>
__device__ __forceinline__ float block_max(float a) {
    __shared__ float sh[NTH / 64];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
    __syncthreads();
    float m = sh[0];
#pragma unroll
    for (int i = 1; i < NTH / 64; i++) m = fmaxf(m, sh[i]);
    return m;
}

typedef float f2vr __attribute__((ext_vector_type(2)));

// CH elements per thread, W = min(block_cols, CH) elements per block in a thread
template <bool BF, int CH, int W>
__global__ __launch_bounds__(NT) void k_rows(QParams p, int amax_only) {
    const Elem E = make_elem(p.elem, p.asym);
    const int64_t cpr = p.cols / CH;
    const int64_t total = p.rows * cpr;
    const int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x;
    const bool active = q < total;
    const int64_t r = active ? q / cpr : 0;
    const int64_t c0 = active ? (q - r * cpr) * CH : 0;

    float x[CH];
    load_chunk<BF, CH>(p, r, c0, active, x);
    if (p.had) hadamard<CH>(x, p.had);

    if (amax_only) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < CH; i++)
            if (finitef(x[i])) a = fmaxf(a, fabsf(x[i]));
        a = block_max<NT>(a);
        if (threadIdx.x == 0) p.amax_parts[blockIdx.x] = a;
        return;
    }

    // macro-block scaling: s_M = UE4M3 rounding of the mantissa of max|x| / Qmax
    float y[CH];
    float sM = 1.0f;
    if (p.macro_cols) {
        const int mg = 128 / CH;
        float M = 0.f;
#pragma unroll
        for (int i = 0; i < CH; i++)
            if (finitef(x[i])) M = fmaxf(M, fabsf(x[i]));
        M = group_max_rt(M, mg);
        int smc = 0x38;
        if (M > 0.f) {
            float t = M / E.qmax;
            float mu = t * pow2f(-flog2(t));
            smc = fp8_code(false, mu);
            sM = fp8_value(false, smc);
        }
        if (active && (threadIdx.x % mg) == 0) p.macro[r * (p.cols / 128) + c0 / 128] = (uint8_t)smc;
#pragma unroll
        for (int i = 0; i < CH; i++) y[i] = x[i] / sM;
    } else {
#pragma unroll
        for (int i = 0; i < CH; i++) y[i] = x[i];
    }

    uint32_t rnd[CH];
    if (p.round == SR) {
        const uint64_t idx0 = (uint64_t)(r * p.cols + c0);
#pragma unroll
        for (int k = 0; k < CH / 8; k++) draws8(p.seed, p.off, (idx0 >> 3) + k, rnd + 8 * k);
    } else {
#pragma unroll
        for (int i = 0; i < CH; i++) rnd[i] = 0;
    }

    const int G = p.bc >= CH ? p.bc / CH : 1;
    const bool leader = (threadIdx.x % G) == 0;
    const float g = (p.scale == SC_NVFP4) ? *p.tensor_scale : 1.0f;
    const int eref = (p.scale == SC_E3M0) ? *p.ref_exp : 0;
    const bool ue5 = p.scale == SC_UE5M3;

    int code[CH];
    float d[CH];
    unsigned long long zb = 0;

#pragma unroll
    for (int j = 0; j < CH / W; j++) {
        float amax = 0.f, mn = INFINITY, mx = -INFINITY;
        int fin = 1;
#pragma unroll
        for (int i = 0; i < W; i++) {
            float v = y[j * W + i];
            if (!finitef(v)) { fin = 0; continue; }
            amax = fmaxf(amax, fabsf(v));
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
        }
        amax = group_max_rt(amax, G);
        fin = group_and_rt(fin, G);
        if (p.asym) {
            mn = group_min_rt(mn, G);
            mx = group_max_rt(mx, G);
        }

        // kind 0: scale 2^e (plus offset o); 1: divide by S; 2: zero scale; 3: non-finite
        int kind = 0, e = 0, sc = 0;
        float S = 1.f, sb = 1.f, o = 0.f;
        uint16_t ob = 0;
        if (!fin) {
            kind = 3;
            sc = nan_scale_code(p.scale);
        } else if (p.asym) {
            if (E.kind == INT4) {
                ob = bf16_floor(mn);
                o = bf16f(ob);
                float R = mx - o;
                e = R > 0.f ? e8m0_exp(p.rule, p.tau, E, R) : -127;
            } else {
                // the mid-range, each end halved first so that it cannot overflow
                ob = bf16_rne(mx * 0.5f + mn * 0.5f);
                o = bf16f(ob);
                float ym = 0.f;
#pragma unroll
                for (int i = 0; i < W; i++) ym = fmaxf(ym, fabsf(y[j * W + i] - o));
                ym = group_max_rt(ym, G);
                e = e8m0_exp(p.rule, p.tau, E, ym);
            }
            sc = e + 127;
        } else if (p.scale == SC_E8M0) {
            e = e8m0_exp(p.rule, p.tau, E, amax);
            sc = e + 127;
        } else if (p.scale == SC_E3M0) {
            int cdown = 7;
            if (amax > 0.f) {
                cdown = eref - e_ceil(amax, E.qmax);
                cdown = cdown < 0 ? 0 : (cdown > 7 ? 7 : cdown);
            }
            e = eref - cdown;
            sc = cdown;
        } else {
            float t = amax / E.qmax;
            if (p.scale == SC_NVFP4) t = t / g;
            sc = fp8_code(ue5, t);
            sb = fp8_value(ue5, sc);
            S = (p.scale == SC_NVFP4) ? sb * g : sb;
            kind = (S == 0.f) ? 2 : 1;
        }

        const float down = pow2f(-e), up = pow2f(e);
        int allzero = 1;
        if (E.kind == E2M1 && p.round == RTNE && kind != 3) {
            // E2M1 to nearest: two elements per hardware convert (RTNE with
            // saturation, signed zero kept) and two per decode; a power-of-two
            // scale decodes as q * 2^e exactly (the convert reads the scale's
            // exponent field; 2^-127 is the zero field)
#pragma unroll
            for (int i = 0; i < W; i += 2) {
                const int k = j * W + i;
                float v[2];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const float yk = y[k + h];
                    if (kind == 0) v[h] = (p.asym ? (yk - o) : yk) * down;
                    else if (kind == 1) v[h] = yk / S;
                    else v[h] = (fbits(yk) >> 31) ? -0.f : 0.f;
                }
                const uint32_t cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
                const f2vr q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, kind == 0 ? up : 1.0f, 0);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    float dv = q[h];
                    if (kind == 0) {
                        if (p.asym) dv = dv + o;
                        if (p.macro_cols) dv = dv * sM;
                    } else {
                        dv = dv * sb;
                        if (p.scale == SC_NVFP4) dv = dv * g;
                    }
                    code[k + h] = (int)((cw >> (4 * h)) & 0xfu);
                    d[k + h] = dv;
                    allzero &= (dv == 0.f);
                }
            }
        } else
#pragma unroll
        for (int i = 0; i < W; i++) {
            const int k = j * W + i;
            float v;
            int c;
            float dv;
            if (kind == 3) {
                c = 0;
                dv = __uint_as_float(0x7fc00000u);
            } else {
                if (kind == 0) v = (p.asym ? (y[k] - o) : y[k]) * down;
                else if (kind == 1) v = y[k] / S;
                else v = (fbits(y[k]) >> 31) ? -0.f : 0.f;
                // E2M1 rows with stochastic rounding and E8M0 scales take the
                // wave-tile kernel unless a dequantized output is asked for
                c = encode<false>(E, kind == 2 ? RTNE : p.round, v, rnd[k]);
                float val = decode(E, c);
                if (kind == 0) {
                    dv = val * up;
                    if (p.asym) dv = dv + o;
                    if (p.macro_cols) dv = dv * sM;
                } else {
                    dv = val * sb;
                    if (p.scale == SC_NVFP4) dv = dv * g;
                }
            }
            code[k] = c;
            d[k] = dv;
            allzero &= (dv == 0.f);
        }
        allzero = group_and_rt(allzero, G);
        if (active && leader) {
            const int64_t sidx = r * (p.cols / p.bc) + (c0 + j * W) / p.bc;
            p.scales[sidx] = (uint8_t)sc;
            if (p.asym) p.offsets[sidx] = kind == 3 ? (uint16_t)0 : ob;
            zb += (unsigned long long)allzero;
        }
    }

    if (active) {
        store_codes(p.codes + r * code_row_bytes(E.bits, p.cols), E.bits, c0, code, CH);
        if (p.dq) store_dq<CH>(p, r, c0, d);
    }
    if (p.parts) {
        // the thread's sums in fp32, then float64 (the whole thread in float64
        // when a square leaves the fp32 range, or a NaN is present)
        double s2 = 0, e2 = 0;
        unsigned long long nz = 0, fl = 0;
        if (active) {
            float s2f = 0.f, e2f = 0.f;
#pragma unroll
            for (int i = 0; i < CH; i++) {
                const float ri = x[i] - d[i];
                s2f = __builtin_fmaf(x[i], x[i], s2f);
                e2f = __builtin_fmaf(ri, ri, e2f);
                nz += (x[i] != 0.f);
                fl += (x[i] != 0.f && d[i] == 0.f);
            }
            if (fabsf(s2f) < INFINITY && fabsf(e2f) < INFINITY) {
                s2 = s2f;
                e2 = e2f;
            } else {
#pragma unroll
                for (int i = 0; i < CH; i++) {
                    const double xv = x[i], dv = d[i];
                    s2 += xv * xv;
                    e2 += (xv - dv) * (xv - dv);
                }
            }
        }
        block_stats<NT>(s2, e2, nz, fl, zb, p.parts + blockIdx.x);
    }
}

}  // namespace

int64_t rows_grid(const QParams& p) {
    const int CH = (p.cols % 16 == 0) ? 16 : 8;
    return (p.rows * (p.cols / CH) + NT - 1) / NT;
}

hipError_t launch_rows(const QParams& p, bool amax_only, hipStream_t s) {
    const int64_t grid = rows_grid(p);
    if (grid == 0) return hipSuccess;
    const bool ch16 = p.cols % 16 == 0;
    const int a = amax_only ? 1 : 0;
    if (p.in_bf16) {
        if (!ch16) k_rows<true, 8, 8><<<grid, NT, 0, s>>>(p, a);
        else if (p.bc == 8 && !amax_only) k_rows<true, 16, 8><<<grid, NT, 0, s>>>(p, a);
        else k_rows<true, 16, 16><<<grid, NT, 0, s>>>(p, a);
    } else {
        if (!ch16) k_rows<false, 8, 8><<<grid, NT, 0, s>>>(p, a);
        else if (p.bc == 8 && !amax_only) k_rows<false, 16, 8><<<grid, NT, 0, s>>>(p, a);
        else k_rows<false, 16, 16><<<grid, NT, 0, s>>>(p, a);
    }
    return hipGetLastError();
}

int64_t amax_grid(const QParams& p) { return std::max(rows_grid(p), rows_fast_grid(p)); }


namespace {

// ---------------------------------------------------------------------------
// MXFP4 fast path: E2M1 elements, E8M0 scales (any exponent rule), round to
// nearest even, dense rows (ld == cols), with or without a dense dequantized
// output (fp32 or bf16, taken from the decode).  gfx950's V_CVT_SCALEF32_PK_FP4_*
// rounds x * 2^-e onto E2M1 with saturation and keeps the sign of zero (two
// elements per instruction, bf16 inputs taken directly); it reads only the
// exponent field of its scale operand, and a zero field means 2^-127, so the
// scale operand is just the E8M0 code shifted into place.  The decode form
// V_CVT_SCALEF32_PK_F32_FP4 gives back value * 2^e.
//
// One "chunk" is 16 bytes of input (8 bf16 or 4 fp32).  A wave tile is 4 x 64
// consecutive chunks; lane l takes chunks l, 64 + l, 128 + l, 192 + l, so each
// of its four loads is one fully coalesced 1 KiB wave-load and a block of b
// elements spans G = b / (elements per chunk) neighbouring lanes.  Waves walk
// the tiles grid-stride; without statistics each loads the next tile before
// working on the current one, with statistics one tile at a time (eight waves
// per SIMD then cover each other's loads).  Every global access goes through a buffer resource that covers just the
// valid part of the tile: reads past the end return zero and writes past it
// are dropped, so the loop has no per-lane bounds branches.
// ---------------------------------------------------------------------------
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s2v __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// a packed pair of bf16 as the operand of the bf16 FP4 convert.  Built by a
// byte copy from a scalar: a __builtin_bit_cast of a component of a
// u32x4 into this operand is miscompiled by this compiler (every convert then
// reads the first component).
__device__ __forceinline__ bf2v as_bf2(uint32_t u) {
    bf2v r;
    __builtin_memcpy(&r, &u, 4);
    return r;
}
// the same for a pair of 16-bit integers (the same miscompile hits this cast)
__device__ __forceinline__ us2 as_us2(uint32_t u) {
    us2 r;
    __builtin_memcpy(&r, &u, 4);
    return r;
}

// raw buffer resource over [base, base + bytes): 32-bit data format, so
// accesses at or beyond `bytes` are out of range (loads give 0, stores drop)
__device__ __forceinline__ rsrc_t buf(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int CPOL_NT = 2;   // non-temporal cache policy of a buffer access
constexpr int OOB_OFFSET = 0x40000000;   // beyond every resource built here

// lane exchanges within a row of 16 lanes (DPP controls)
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <- lane 15 - i
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- lane 7 - i within each 8

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    // every lane has a source under these controls; the zero "old" value lets
    // the compiler fold the move into the consuming max
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// maximum over aligned groups of G neighbouring lanes, the result
// in every lane of the group.  After the two quad steps every quad holds its
// value; the half-row mirror pairs the two quads of an 8-lane group, the row
// mirror the two halves of a 16-lane row; wider groups use cross-row shuffles.
template <int G>
__device__ __forceinline__ uint32_t group_max_u(uint32_t v) {
    if constexpr (G >= 2) v = max(v, dpp<DPP_XOR1>(v));
    if constexpr (G >= 4) v = max(v, dpp<DPP_XOR2>(v));
    if constexpr (G >= 8) v = max(v, dpp<DPP_HALF_MIRROR>(v));
    if constexpr (G >= 16) v = max(v, dpp<DPP_ROW_MIRROR>(v));
    if constexpr (G >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if constexpr (G >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}

// E8M0 exponent of a finite block maximum given by its float bits u (sign
// clear), clamped to [-127, 127]; u = 0 lands on -127.
//   FLOOR:      floor(log2 amax) - 2, 2 being E2M1's largest exponent
//   CEIL, OAS:  the smallest e with q * 2^e >= amax, where q = 2^lq * (1 + fq/2^23)
//               is 6 (CEIL) or tau (OAS): compare exponents, then significands.
template <bool FLOOR>
__device__ __forceinline__ int fast_exp(uint32_t u, int lq, uint32_t fq) {
    const int be = (int)(u >> 23);
    const int lz = __clz(u);                       // 32 for u = 0
    const int lg = be ? be - 127 : -118 - lz;      // floor(log2), subnormals included
    int e;
    if constexpr (FLOOR) {
        e = lg - 2;
    } else {
        const uint32_t fr = be ? (u & 0x7fffffu) : ((u << ((lz - 8) & 31)) & 0x7fffffu);
        e = lg - lq + (fr > fq ? 1 : 0);
    }
    return min(max(e, -127), 127);
}

constexpr int FAST_NL = 4;                 // chunks per lane per wave tile
constexpr int TILE_CH = 64 * FAST_NL;      // chunks per wave tile
constexpr int64_t FAST_MAX_GRID = 2048;
#ifndef FAST_WAVES
#define FAST_WAVES 6   // waves per SIMD the register budget is sized for
#endif

// One tensor's share of a launch: workgroup blk of nblk walks the tiles of
// x (nchunks chunks) grid-stride and writes its codes, scales, (ST) one
// statistics partial at parts[blk] and (DQ) the dequantized values to dq,
// dense, fp32 or (dq_bf16) bf16.
template <bool BF, int G, bool FLOOR, bool ST, bool DQ = false>
__device__ __forceinline__ void rows_fast_run(const void* x, uint8_t* codes, uint8_t* scales, StatPart* parts,
                                              int64_t nchunks, int lq, uint32_t fq, int64_t blk, int64_t nblk,
                                              void* dq = nullptr, int dq_bf16 = 0) {
    constexpr int EPC = BF ? 8 : 4;        // elements per chunk
    constexpr int CB = EPC / 2;            // code bytes per chunk
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (nchunks + TILE_CH - 1) / TILE_CH;
    const int64_t step = nblk * (NT / 64);
    const char* xin = static_cast<const char*>(x);
    // per-lane buffer offsets; the per-chunk parts are constants that go into the
    // instructions' offset fields.  A block's scale byte is stored by its first
    // lane; the others aim past the resource and the store drops them (no
    // branch, so a chunk stays one basic block).
    const int lin = lane * 16, lco = lane * CB;
    const int lsc = lane % G == 0 ? lane / G : OOB_OFFSET;
    const uint32_t lead = lane % G == 0 ? 1u : 0u;
    double s2d = 0.0, e2d = 0.0;
    uint32_t nz = 0, fl = 0, zb = 0;

    // valid chunks of tile t (0 past the end)
    auto valid = [&](int64_t t) -> int {
        const int64_t r = nchunks - t * TILE_CH;
        return r <= 0 ? 0 : (r < TILE_CH ? (int)r : TILE_CH);
    };
    auto load = [&](u32x4* w, int64_t t) {
        const rsrc_t r = buf(xin + t * TILE_CH * 16, valid(t) * 16);
#pragma unroll
        for (int k = 0; k < FAST_NL; k++)
            w[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lin + k * 1024, 0, CPOL_NT));
    };

    auto work = [&](const u32x4* w, int64_t t) {
        const int nv = valid(t);
        const rsrc_t rc = buf(codes + t * TILE_CH * CB, nv * CB);
        const rsrc_t rs = buf(scales + t * (TILE_CH / G), nv / G);
        // (DQ) the tile's dequantized output: EPC values of 4 or 2 bytes per chunk
        const int dqb = dq_bf16 ? 2 : 4;
        const rsrc_t rdq = buf(DQ ? static_cast<char*>(dq) + t * TILE_CH * EPC * dqb : static_cast<char*>(nullptr),
                               DQ ? nv * EPC * dqb : 0);
        float s2 = 0.f, e2 = 0.f;
#pragma unroll
        for (int k = 0; k < FAST_NL; k++) {
            // |x| with the sign bits cleared, and the block maximum of it: for bf16
            // the 15-bit magnitude, for fp32 the float bits
            u32x4 t4;
            uint32_t am;
            if constexpr (BF) {
                t4 = w[k] & 0x7fff7fffu;
                const us2 m = __builtin_elementwise_max(__builtin_elementwise_max(as_us2(t4.x), as_us2(t4.y)),
                                                        __builtin_elementwise_max(as_us2(t4.z), as_us2(t4.w)));
                am = max((uint32_t)m[0], (uint32_t)m[1]);
            } else {
                t4 = w[k] & 0x7fffffffu;
                am = max(max(t4.x, t4.y), max(t4.z, t4.w));
            }
            am = group_max_u<G>(am);
            const uint32_t ab = BF ? am << 16 : am;   // as float bits
            const bool nonfinite = ab >= 0x7f800000u;
            // scale operand of the converts: the E8M0 code in the exponent field.
            // FLOOR: code = biased exponent of amax - 2, floored at 0 (a saturating
            // subtract; zero and subnormal maxima land on code 0 as well)
            uint32_t sbits;
            if constexpr (FLOOR) sbits = __builtin_elementwise_sub_sat(ab & 0x7f800000u, 0x01000000u);
            else sbits = (uint32_t)(fast_exp<false>(ab, lq, fq) + 127) << 23;
            const uint32_t code = sbits >> 23;
            const float scale = __uint_as_float(sbits);
            uint32_t cw = 0;
            if constexpr (BF) {
                const uint32_t a0 = w[k][0], a1 = w[k][1], a2 = w[k][2], a3 = w[k][3];
                cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(cw, as_bf2(a0), scale, 0);
                cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(cw, as_bf2(a1), scale, 1);
                cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(cw, as_bf2(a2), scale, 2);
                cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(cw, as_bf2(a3), scale, 3);
            } else {
                cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, __uint_as_float(w[k].x), __uint_as_float(w[k].y), scale, 0);
                cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, __uint_as_float(w[k].z), __uint_as_float(w[k].w), scale, 1);
            }
            if (nonfinite) cw = 0;
            if constexpr (BF) __builtin_amdgcn_raw_buffer_store_b32(cw, rc, lco + k * 64 * CB, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)cw, rc, lco + k * 64 * CB, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(nonfinite ? 0xffu : code), rs, lsc + k * (64 / G), 0, 0);

            // dequantized values straight from the codes (value * 2^e)
            float d[EPC];
            if constexpr (ST || DQ) {
                f2v dd[EPC / 2];
                dd[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 0);
                dd[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 1);
                if constexpr (BF) {
                    dd[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 2);
                    dd[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 3);
                }
#pragma unroll
                for (int j = 0; j < EPC / 2; j++) { d[2 * j] = dd[j][0]; d[2 * j + 1] = dd[j][1]; }
            }
            if constexpr (DQ) {
                // a non-finite block dequantizes to NaN; bf16 keeps the upper half
                // of each value, which is exact (E2M1 values carry 2 significant bits)
                u32x4 o0, o1;
                const uint32_t qn = 0x7fc00000u;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    o0[j] = nonfinite ? qn : __float_as_uint(d[j]);
                    if constexpr (BF) o1[j] = nonfinite ? qn : __float_as_uint(d[4 + j]);
                }
                if (dq_bf16) {
                    u32x4 b;
                    b[0] = (o0[0] >> 16) | (o0[1] & 0xffff0000u);
                    b[1] = (o0[2] >> 16) | (o0[3] & 0xffff0000u);
                    if constexpr (BF) {
                        b[2] = (o1[0] >> 16) | (o1[1] & 0xffff0000u);
                        b[3] = (o1[2] >> 16) | (o1[3] & 0xffff0000u);
                        __builtin_amdgcn_raw_buffer_store_b128(b, rdq, lane * 16 + k * 1024, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b64((u32x2){b[0], b[1]}, rdq, lane * 8 + k * 512, 0, 0);
                    }
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128(o0, rdq, lane * (EPC * 4) + k * 64 * (EPC * 4), 0, 0);
                    if constexpr (BF)
                        __builtin_amdgcn_raw_buffer_store_b128(o1, rdq, lane * 32 + 16 + k * 64 * 32, 0, 0);
                }
            }
            if constexpr (ST) {
                // A zero input always gets a zero code, so flushed = #zero-magnitude
                // codes - #zero inputs (NaN and Inf count as nonzero; a non-finite
                // block flushes nothing).  Chunks past the end read as zeros and
                // contribute nothing, except to the all-zero-block count, which
                // checks the block's position.  A block is all zero codes iff its
                // maximum rounds to a zero code.
                const uint32_t ca = BF ? __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, as_bf2(am), scale, 0)
                                       : __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __uint_as_float(am), 0.f, scale, 0);
                const uint32_t allz = (!nonfinite && (ca & 7u) == 0) ? 1u : 0u;
                // nonzero inputs: adding 0x7fff to a 15-bit magnitude sets bit 15 iff
                // it is nonzero; a byte permute gathers the four flag bytes of two
                // words, then the flags are counted
                uint32_t nzc;
                if constexpr (BF) {
                    const uint32_t f0 = t4.x + 0x7fff7fffu, f1 = t4.y + 0x7fff7fffu;
                    const uint32_t f2 = t4.z + 0x7fff7fffu, f3 = t4.w + 0x7fff7fffu;
                    const uint32_t g01 = __builtin_amdgcn_perm(f0, f1, 0x07050301u) & 0x80808080u;
                    const uint32_t g23 = __builtin_amdgcn_perm(f2, f3, 0x07050301u) & 0x80808080u;
                    nzc = __builtin_popcount(g01) + __builtin_popcount(g23);
                } else {
                    nzc = min(t4.x, 1u) + min(t4.y, 1u) + min(t4.z, 1u) + min(t4.w, 1u);
                }
                const uint32_t tm = cw & (BF ? 0x77777777u : 0x7777u);
                const uint32_t zc = __builtin_popcount(~(tm + (BF ? 0x77777777u : 0x7777u)) &
                                                       (BF ? 0x88888888u : 0x8888u));
                nz += nzc;
                fl += nonfinite ? 0u : zc - (EPC - nzc);
                zb += allz & lead & (lane + k * 64 < nv ? 1u : 0u);
                if constexpr (BF) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const uint32_t wj = w[k][j];
                        s2 = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wj), as_bf2(wj), s2, false);
                        const float r0 = __uint_as_float(wj << 16) - d[2 * j];
                        const float r1 = __uint_as_float(wj & 0xffff0000u) - d[2 * j + 1];
                        e2 = __builtin_fmaf(r0, r0, e2);
                        e2 = __builtin_fmaf(r1, r1, e2);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const float xj = __uint_as_float(w[k][j]), r = xj - d[j];
                        s2 = __builtin_fmaf(xj, xj, s2);
                        e2 = __builtin_fmaf(r, r, e2);
                    }
                }
                if (nonfinite) e2 = __uint_as_float(0x7fc00000u);
            }
            // keep the chunks in order: interleaving all of them costs registers, not time
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ST) {
            s2d += (double)s2;
            e2d += (double)e2;
        }
    };

    if constexpr (ST) {
        // with statistics: one register tile, so that the kernel fits 64
        // registers and 8 waves per SIMD hide each other's loads (measured 3%
        // faster than the ping-pong below at 6 waves)
        for (int64_t t = blk * (NT / 64) + wave; t < ntiles; t += step) {
            u32x4 w1[FAST_NL];
            load(w1, t);
            work(w1, t);
        }
    } else {
        // two register tiles in ping-pong: one is worked on while the other loads
        int64_t t = blk * (NT / 64) + wave;
        u32x4 wa[FAST_NL], wb[FAST_NL];
        load(wa, t);
        while (t < ntiles) {
            load(wb, t + step);
            work(wa, t);
            t += step;
            if (t >= ntiles) break;
            load(wa, t + step);
            work(wb, t);
            t += step;
        }
    }
    if constexpr (ST) block_stats<NT>(s2d, e2d, nz, fl, zb, parts + blk);
}

// waves per SIMD the register budget is sized for: 8 with statistics only
// (64 registers, so the waves cover each other's loads), fewer otherwise, and
// 4 for statistics with a dequantized output (128 registers, no spills)
#define MX_FAST_ATTRS(DQv)                                                                                  \
    __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(                                               \
        (G >= 32 || (ST && (DQv))) ? 4 : (FLOOR ? ((ST && !(DQv)) ? 8 : FAST_WAVES) : FAST_WAVES - 1), 8)))

template <bool BF, int G, bool FLOOR, bool ST, bool DQ>
__global__ MX_FAST_ATTRS(DQ) void k_rows_fast(QParams p, int64_t nchunks, int lq, uint32_t fq) {
    rows_fast_run<BF, G, FLOOR, ST, DQ>(p.x, p.codes, p.scales, p.parts, nchunks, lq, fq, blockIdx.x, gridDim.x,
                                        p.dq, p.dq_bf16);
}

// Several tensors in one launch: tensor i takes the nb workgroups from b0 on
// (the b0 increase with i; a workgroup finds its tensor by a scalar search).
template <bool BF, int G, bool FLOOR, bool ST>
__global__ MX_FAST_ATTRS(false) void k_rows_fast_many(FastMany m, int lq, uint32_t fq) {
    const int64_t b = blockIdx.x;
    int i = 0;
    for (int k = 1; k < m.count; k++)
        if (b >= m.job[k].b0) i = k;
    const FastJob& J = m.job[i];
    rows_fast_run<BF, G, FLOOR, ST>(J.x, J.codes, J.scales, J.parts, J.nchunks, lq, fq, b - J.b0, J.nb);
}
#undef MX_FAST_ATTRS

// ---------------------------------------------------------------------------
// MXFP8 fast path: E4M3 or (E5) E5M2 elements, E8M0 scales (any exponent
// rule), round to nearest even, dense rows; the wave tile and buffer I/O of
// k_rows_fast, one code byte per element.  V_CVT_SCALEF32_PK_FP8_F32 /
// _PK_BF8_F32 round x * 2^-e to nearest even but do not saturate (an overflow
// gives the NaN / Inf code), so each element is first clamped to +-Qmax 2^e:
// exact, and the rounding then gives Qmax for every larger magnitude, the
// format's saturation.  The decode forms give back value * 2^e.
// ---------------------------------------------------------------------------
template <bool E5>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w, float a, float b, float scale, bool hi) {
    s2v r;
    __builtin_memcpy(&r, &w, 4);
    r = hi ? (E5 ? __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, a, b, scale, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, scale, true))
           : (E5 ? __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, a, b, scale, false)
                 : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, scale, false));
    uint32_t o;
    __builtin_memcpy(&o, &r, 4);
    return o;
}

template <bool E5>
__device__ __forceinline__ f2v fp8_unpair(uint32_t w, float scale, bool hi) {
    return hi ? (E5 ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, scale, true)
                    : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, true))
              : (E5 ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, scale, false)
                    : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, false));
}

// ---------------------------------------------------------------------------
// MXFP6 fast path: E2M3 or (E3) E3M2 elements, E8M0 scales (any exponent
// rule) on 1 x 32 blocks, round to nearest even, dense rows.  The FP6 pack
// converts take a whole block from one lane: V_CVT_SCALEF32_PK32_FP6_BF16 /
// _BF6_BF16 its 32 bf16 values, V_CVT_SCALEF32_2XPK16_FP6_F32 / _BF6_F32 its
// 32 fp32 values as the even and the odd ones (element 2i from the first
// operand, 2i + 1 from the second), and both round x * 2^-e to nearest even
// with saturation into the 24-byte least-significant-bit-first code stream
// of the block.  So lane l takes block l of a 64-block wave tile (64 or 128
// contiguous bytes of input), and the decode gives the 32 values back times 2^e.
// ---------------------------------------------------------------------------
typedef __bf16 bf32v __attribute__((ext_vector_type(32)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f32v __attribute__((ext_vector_type(32)));
typedef uint32_t u6v __attribute__((ext_vector_type(6)));
constexpr int FP6_TILE = 64 * 32;          // elements per wave tile

template <bool BF, bool ST, bool E3>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_rows_fp6(QParams p, int64_t nelem,
                                                                                          int lq, uint32_t fq,
                                                                                          int floor_rule) {
    constexpr int NL = BF ? 4 : 8;         // 16-byte loads per lane (one block)
    constexpr int EMAX = E3 ? 4 : 2;       // floor(log2 Qmax)
    const bool DQ = p.dq != nullptr;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (nelem + FP6_TILE - 1) / FP6_TILE;
    const int64_t step = (int64_t)gridDim.x * (NT / 64);
    const char* xin = static_cast<const char*>(p.x);
    double s2d = 0.0, e2d = 0.0;
    uint32_t nz = 0, fl = 0, zb = 0;
    for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + wave; t < ntiles; t += step) {
        const int64_t r = nelem - t * FP6_TILE;
        const int ne = r < FP6_TILE ? (int)r : FP6_TILE;   // a multiple of 32
        const rsrc_t rx = buf(xin + t * FP6_TILE * (BF ? 2 : 4), ne * (BF ? 2 : 4));
        const rsrc_t rc = buf(p.codes + t * FP6_TILE * 3 / 4, ne * 3 / 4);
        const rsrc_t rs = buf(p.scales + t * 64, ne / 32);
        const int dqb = p.dq_bf16 ? 2 : 4;
        const rsrc_t rdq = buf(DQ ? static_cast<char*>(p.dq) + t * FP6_TILE * dqb : static_cast<char*>(nullptr),
                               DQ ? ne * dqb : 0);
        u32x4 w[NL];
#pragma unroll
        for (int k = 0; k < NL; k++)
            w[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, lane * (NL * 16) + k * 16, 0, 0));
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const uint32_t wi = w[BF ? i / 8 : i / 4][BF ? (i / 2) % 4 : i % 4];
            x[i] = BF ? ((i & 1) ? bf16hi(wi) : bf16lo(wi)) : __uint_as_float(wi);
        }
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 32; i++) am = max(am, __float_as_uint(x[i]) & 0x7fffffffu);
        const bool nonfinite = am >= 0x7f800000u;
        uint32_t sbits;
        if (floor_rule) sbits = __builtin_elementwise_sub_sat(am & 0x7f800000u, (uint32_t)EMAX << 23);
        else sbits = (uint32_t)(fast_exp<false>(am, lq, fq) + 127) << 23;
        const uint32_t code = sbits >> 23;
        const float scale = __uint_as_float(sbits);
        u6v cw;
        if constexpr (BF) {
            bf32v vb;
            __builtin_memcpy(&vb, w, 64);
            cw = E3 ? __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(vb, scale)
                    : __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(vb, scale);
        } else {
            f16v ev, od;
#pragma unroll
            for (int i = 0; i < 16; i++) { ev[i] = x[2 * i]; od[i] = x[2 * i + 1]; }
            cw = E3 ? __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, scale)
                    : __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, scale);
        }
        if (nonfinite) cw = (u6v){0u, 0u, 0u, 0u, 0u, 0u};
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){cw[0], cw[1], cw[2], cw[3]}, rc, lane * 24, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){cw[4], cw[5]}, rc, lane * 24 + 16, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(nonfinite ? 0xffu : code), rs, lane, 0, 0);
        if (ST || DQ) {
            const f32v dv = E3 ? __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(cw, scale)
                               : __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(cw, scale);
            if (DQ) {
                // a non-finite block dequantizes to NaN; bf16 keeps the upper half of
                // each value, which is exact (FP6 values carry 4 or 3 significant bits)
                uint32_t o[32];
#pragma unroll
                for (int i = 0; i < 32; i++) o[i] = nonfinite ? 0x7fc00000u : __float_as_uint(dv[i]);
                if (p.dq_bf16) {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        u32x4 b;
#pragma unroll
                        for (int j = 0; j < 4; j++) b[j] = (o[8 * q + 2 * j] >> 16) | (o[8 * q + 2 * j + 1] & 0xffff0000u);
                        __builtin_amdgcn_raw_buffer_store_b128(b, rdq, lane * 64 + q * 16, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 8; q++)
                        __builtin_amdgcn_raw_buffer_store_b128((u32x4){o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]},
                                                               rdq, lane * 128 + q * 16, 0, 0);
                }
            }
            if constexpr (ST) {
                // lanes past the end read zeros and count only for the zero blocks
                const bool valid = lane * 32 < ne;
                float s2 = 0.f, e2 = 0.f;
                uint32_t anyd = 0;
#pragma unroll
                for (int i = 0; i < 32; i++) {
                    const float ri = x[i] - dv[i];
                    s2 = __builtin_fmaf(x[i], x[i], s2);
                    e2 = __builtin_fmaf(ri, ri, e2);
                    nz += x[i] != 0.f ? 1u : 0u;
                    fl += (!nonfinite && x[i] != 0.f && dv[i] == 0.f) ? 1u : 0u;
                    anyd |= dv[i] != 0.f ? 1u : 0u;
                }
                zb += (valid && !nonfinite && anyd == 0) ? 1u : 0u;
                if (fabsf(s2) < INFINITY && !nonfinite) {
                    s2d += (double)s2;
                    e2d += (double)e2;
                } else {
                    // a square beyond the fp32 range, or a NaN / Inf: this block in float64
#pragma unroll
                    for (int i = 0; i < 32; i++) {
                        const double xd = x[i], dd = nonfinite ? (double)__uint_as_float(0x7fc00000u) : (double)dv[i];
                        s2d += xd * xd;
                        e2d += (xd - dd) * (xd - dd);
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ST) block_stats<NT>(s2d, e2d, nz, fl, zb, p.parts + blockIdx.x);
}

// floor_rule and the dequantized output (p.dq) are uniform run-time switches
template <bool BF, int G, bool ST, bool E5>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_rows_fp8(QParams p, int64_t nchunks,
                                                                                          int lq, uint32_t fq,
                                                                                          int floor_rule) {
    const bool DQ = p.dq != nullptr;
    constexpr int EPC = BF ? 8 : 4;        // elements (and code bytes) per chunk
    constexpr int EMAX = E5 ? 15 : 8;      // floor(log2 Qmax); Qmax = 1.75 x 2^EMAX
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (nchunks + TILE_CH - 1) / TILE_CH;
    const int64_t step = (int64_t)gridDim.x * (NT / 64);
    const char* xin = static_cast<const char*>(p.x);
    const int lin = lane * 16, lco = lane * EPC;
    const int lsc = lane % G == 0 ? lane / G : OOB_OFFSET;
    const uint32_t lead = lane % G == 0 ? 1u : 0u;
    double s2d = 0.0, e2d = 0.0;
    uint32_t nz = 0, fl = 0, zb = 0;
    for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + wave; t < ntiles; t += step) {
        const int64_t r = nchunks - t * TILE_CH;
        const int nv = r < TILE_CH ? (int)r : TILE_CH;
        const rsrc_t rx = buf(xin + t * TILE_CH * 16, nv * 16);
        const rsrc_t rc = buf(p.codes + t * TILE_CH * EPC, nv * EPC);
        const rsrc_t rs = buf(p.scales + t * (TILE_CH / G), nv / G);
        const int dqb = p.dq_bf16 ? 2 : 4;
        const rsrc_t rdq = buf(DQ ? static_cast<char*>(p.dq) + t * TILE_CH * EPC * dqb : static_cast<char*>(nullptr),
                               DQ ? nv * EPC * dqb : 0);
        u32x4 w[FAST_NL];
#pragma unroll
        for (int k = 0; k < FAST_NL; k++)
            w[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, lin + k * 1024, 0, CPOL_NT));
#pragma unroll
        for (int k = 0; k < FAST_NL; k++) {
            float x[EPC];
#pragma unroll
            for (int i = 0; i < EPC; i++)
                x[i] = BF ? ((i & 1) ? bf16hi(w[k][i >> 1]) : bf16lo(w[k][i >> 1])) : __uint_as_float(w[k][i]);
            uint32_t am = 0;
#pragma unroll
            for (int i = 0; i < EPC; i++) am = max(am, __float_as_uint(x[i]) & 0x7fffffffu);
            am = group_max_u<G>(am);
            const bool nonfinite = am >= 0x7f800000u;
            uint32_t sbits;
            if (floor_rule) sbits = __builtin_elementwise_sub_sat(am & 0x7f800000u, (uint32_t)EMAX << 23);
            else sbits = (uint32_t)(fast_exp<false>(am, lq, fq) + 127) << 23;
            const uint32_t code = sbits >> 23;
            const float scale = __uint_as_float(sbits);
            // Qmax 2^e = 1.75 x 2^(e + EMAX); beyond the fp32 range no element can exceed it
            const float c = __uint_as_float(code + EMAX >= 255 ? 0x7f800000u : ((code + EMAX) << 23) | 0x600000u);
            uint32_t cw[EPC / 4];
#pragma unroll
            for (int q = 0; q < EPC / 4; q++) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; i++) v[i] = __builtin_amdgcn_fmed3f(x[4 * q + i], -c, c);
                uint32_t u = fp8_pair<E5>(0u, v[0], v[1], scale, false);
                cw[q] = nonfinite ? 0u : fp8_pair<E5>(u, v[2], v[3], scale, true);
            }
            if constexpr (BF) __builtin_amdgcn_raw_buffer_store_b64((u32x2){cw[0], cw[1]}, rc, lco + k * 64 * EPC, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b32(cw[0], rc, lco + k * 64 * EPC, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(nonfinite ? 0xffu : code), rs, lsc + k * (64 / G), 0, 0);
            float d[EPC];
            if (ST || DQ) {
#pragma unroll
                for (int q = 0; q < EPC / 4; q++) {
                    const f2v lo = fp8_unpair<E5>(cw[q], scale, false), hi = fp8_unpair<E5>(cw[q], scale, true);
                    d[4 * q] = lo[0]; d[4 * q + 1] = lo[1]; d[4 * q + 2] = hi[0]; d[4 * q + 3] = hi[1];
                }
            }
            if (DQ) {
                // a non-finite block dequantizes to NaN; bf16 keeps the upper half
                // of each value, which is exact (FP8 values carry 4 or 3 significant bits)
                uint32_t o[EPC];
#pragma unroll
                for (int i = 0; i < EPC; i++) o[i] = nonfinite ? 0x7fc00000u : __float_as_uint(d[i]);
                if (p.dq_bf16) {
                    uint32_t b[EPC / 2];
#pragma unroll
                    for (int j = 0; j < EPC / 2; j++) b[j] = (o[2 * j] >> 16) | (o[2 * j + 1] & 0xffff0000u);
                    if constexpr (BF)
                        __builtin_amdgcn_raw_buffer_store_b128((u32x4){b[0], b[1], b[2], b[3]}, rdq, lane * 16 + k * 1024, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b64((u32x2){b[0], b[1]}, rdq, lane * 8 + k * 512, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128((u32x4){o[0], o[1], o[2], o[3]}, rdq,
                                                           lane * (EPC * 4) + k * 64 * (EPC * 4), 0, 0);
                    if constexpr (BF)
                        __builtin_amdgcn_raw_buffer_store_b128((u32x4){o[4], o[5], o[6], o[7]}, rdq,
                                                               lane * 32 + 16 + k * 64 * 32, 0, 0);
                }
            }
            if constexpr (ST) {
                // a block is all zero codes iff its (clamped) maximum rounds to a
                // zero code; chunks past the end read as zeros and count only there
                const float amc = __builtin_amdgcn_fmed3f(__uint_as_float(am), -c, c);
                const uint32_t ca = fp8_pair<E5>(0u, amc, 0.f, scale, false);
                const uint32_t allz = (!nonfinite && (ca & 0x7fu) == 0) ? 1u : 0u;
                float s2 = 0.f, e2 = 0.f;
#pragma unroll
                for (int i = 0; i < EPC; i++) {
                    const float ri = x[i] - d[i];
                    s2 = __builtin_fmaf(x[i], x[i], s2);
                    e2 = __builtin_fmaf(ri, ri, e2);
                    nz += x[i] != 0.f ? 1u : 0u;
                    fl += (!nonfinite && x[i] != 0.f && d[i] == 0.f) ? 1u : 0u;
                }
                zb += allz & lead & (lane + k * 64 < nv ? 1u : 0u);
                if (nonfinite) e2 = __uint_as_float(0x7fc00000u);
                if (fabsf(s2) < INFINITY && !nonfinite) {
                    s2d += (double)s2;
                    e2d += (double)e2;
                } else {
#pragma unroll
                    for (int i = 0; i < EPC; i++) {
                        const double xd = x[i], dd = nonfinite ? (double)__uint_as_float(0x7fc00000u) : (double)d[i];
                        s2d += xd * xd;
                        e2d += (xd - dd) * (xd - dd);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (ST) block_stats<NT>(s2d, e2d, nz, fl, zb, p.parts + blockIdx.x);
}

// ---------------------------------------------------------------------------
// Wave-tile row kernel for the other dense row formats: E2M1 under UE4M3 /
// UE5M3 / NVFP4, E8M0 or E3M0 block scales, with block Hadamard rotation
// ("Bridging the Gap ... Microscaling FP4 Quantization", Sec. 2.2) or
// macro-block scaling ("Unveiling the Potential of Quantization with MXFP4",
// Sec. 4), to nearest or (E8M0 scales) stochastically; INT4, plain or min/max,
// under E8M0 scales to nearest (the ARITH 2025 MX-training report's
// asymmetric INT4).  Dense rows, optional dense dequantized output.  Wave tile, buffer
// I/O and grid-stride loop as in k_rows_fast; the lane groups (scale block: g
// lanes, rotation chunk: hg, macro block: mg) are uniform run-time sizes.
//  - rotation: the butterflies of a chunk's EPC elements in registers, then
//    one stage per lane bit with the partner lane's value (DPP for lane
//    distances 1 and 2, ds_swizzle beyond), in the definition's stage order;
//    the upper lane of a pair forms partner - own as fma(own, -1, partner),
//    which is the same single rounding; then times the fp32 1/sqrt(h);
//  - macro scale: the finite maximum over mg lanes, s_M = UE4M3 rounding of
//    the significand of M / 6; the elements are divided by s_M;
//  - E8M0 scales: the scaled FP4 convert divides by the power of two itself
//    (it reads the exponent field of the scale operand); fp8 scales: the
//    elements are divided by S (correctly rounded) and converted unscaled;
//    E3M0 scales: the elements times 2^-e, converted unscaled;
//  - stochastic rounding: one Philox call per 8 elements at their linear
//    indices, the E2M1 code decided from the bits of the scaled value;
//  - INT4: the integer nearest the scaled value (ties to even), capped; the
//    min/max variant subtracts the bf16 offset first and stores it per block;
//  - decode by the matching FP4 -> f32 convert, times s_b (and g) or s_M
//    (INT4: the integer times 2^e, plus the offset).
// ---------------------------------------------------------------------------
struct HwArgs {
    int64_t nchunks;
    int g, hg, mg;           // lanes per scale block, rotation chunk, macro block (0: none)
    int floor_rule;          // E8M0: FLOOR, else the smallest e with q 2^e >= amax
    int lq;                  // q = 2^lq (1 + fq 2^-23): 6 (CEIL) or tau (OAS)
    uint32_t fq;
    int ue5, nvfp4;          // fp8 scales: UE5M3, NVFP4 (UE4M3 times the tensor scale)
    float hconst;            // fp32 rounding of 1 / sqrt(h)
    int sr;                  // E8M0 scales: stochastic rounding instead of to nearest
    int e3m0;                // E3M0 scales: a step-down below the tensor's reference exponent
    int int4, asym;          // INT4 elements (E8M0 scales, to nearest), the min/max variant
};

// a / b rounded to nearest even, given r = the correctly rounded 1 / b:
// Markstein's correction step, q = a r, e = a - q b (exact, one FMA), then
// q + e r.  It is the correctly rounded quotient whenever no intermediate
// leaves the normal range: for |a| >= 2^-96 and a quotient in [2^-96, 2^120]
// (a block's quotients never exceed max(8, amax / 448); by the macro scales
// 1 .. 2 over the whole range); smaller quotients keep their sign and stay
// below 2^-80, far under any E2M1 rounding point.  The sign of a zero is a's.
// tests/test_division_identity.py emulates the sequence exactly and checks it
// against every finite bf16 input and every UE4M3 / UE5M3 and macro divisor.
__device__ __forceinline__ float div_by(float a, float b, float r) {
    const float q = a * r;
    const float e = __builtin_fmaf(-q, b, a);
    return __builtin_copysignf(__builtin_fmaf(e, r, q), a);
}
// true in every lane when some lane's value is nonzero and below 2^-96, or
// not finite: the chunk then divides exactly
// (the magnitudes' minimum after u - 1, which wraps zero to the top, finds a
// nonzero one below 2^-96; their maximum finds a non-finite one)
template <int N>
__device__ __forceinline__ bool wave_needs_exact_div(const float (&v)[N]) {
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const uint32_t u = __float_as_uint(v[i]) & 0x7fffffffu;
        lo = min(lo, u - 1u);
        hi = max(hi, u);
    }
    return __any(lo < 0x0f7fffffu || hi >= 0x7f800000u);
}

// a / b rounded to nearest even for one value per lane, through div_by with
// r = RN(1/b) when every lane's dividend is zero, not finite, or in [2^-90,
// 2^119] with RN(a r) in [2^-94, 2^118] (then the quotient lies inside
// div_by's range), else by the exact divide
__device__ __forceinline__ float div_lane(float a, float b, float r) {
    const uint32_t u = __float_as_uint(a) & 0x7fffffffu;
    const uint32_t q = __float_as_uint(a * r) & 0x7fffffffu;
    const bool ok = u == 0u || u >= 0x7f800000u ||
                    (u >= 0x12800000u && u <= 0x7b000000u && q >= 0x10800000u && q <= 0x7a800000u);
    if (__all(ok)) return div_by(a, b, r);
    return a / b;
}

// the value of lane l ^ S of the wave (S a power of two below 32)
template <int S>
__device__ __forceinline__ float xlane(float v) {
    const uint32_t u = __float_as_uint(v);
    if constexpr (S == 1) return __uint_as_float(dpp<DPP_XOR1>(u));
    else if constexpr (S == 2) return __uint_as_float(dpp<DPP_XOR2>(u));
    else return __uint_as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)u, 0x1f | (S << 10)));
}

// NP pairs of fp32 values to E2M1 codes (pair i in byte i): the scaled convert
// (round to nearest even, saturating, divided by the power of two whose
// exponent field `scale` carries); and the codes back to values times it
template <int NP>
__device__ __forceinline__ uint32_t enc_fp4(const float* v, float scale) {
    uint32_t cw = 0;
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[0], v[1], scale, 0);
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[2], v[3], scale, 1);
    if constexpr (NP == 4) {
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[4], v[5], scale, 2);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[6], v[7], scale, 3);
    }
    return cw;
}
template <int NP>
__device__ __forceinline__ void dec_fp4(uint32_t cw, float scale, float* d) {
    f2v q[NP];
    q[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 0);
    q[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 1);
    if constexpr (NP == 4) {
        q[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 2);
        q[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 3);
    }
#pragma unroll
    for (int i = 0; i < NP; i++) { d[2 * i] = q[i][0]; d[2 * i + 1] = q[i][1]; }
}

// one rotation stage across lanes at distance S: lower lane a + b, upper a - b
template <int S, int EPC>
__device__ __forceinline__ void had_stage(float (&x)[EPC], int lane) {
    const float sg = (lane & S) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < EPC; i++) x[i] = __builtin_fmaf(x[i], sg, xlane<S>(x[i]));
}

// maximum over aligned groups of g lanes (g uniform, a power of two <= 64)
__device__ __forceinline__ uint32_t group_max_g(uint32_t v, int g) {
    if (g >= 2) v = max(v, dpp<DPP_XOR1>(v));
    if (g >= 4) v = max(v, dpp<DPP_XOR2>(v));
    if (g >= 8) v = max(v, dpp<DPP_HALF_MIRROR>(v));
    if (g >= 16) v = max(v, dpp<DPP_ROW_MIRROR>(v));
    if (g >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if (g >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}

// the minimum (MAXV false) or maximum of a float over aligned groups of g
// lanes, by the lane moves of group_max_g
template <bool MAXV>
__device__ __forceinline__ float group_fext_g(float v, int g) {
    auto op = [](float a, uint32_t b) { return MAXV ? fmaxf(a, __uint_as_float(b)) : fminf(a, __uint_as_float(b)); };
    if (g >= 2) v = op(v, dpp<DPP_XOR1>(__float_as_uint(v)));
    if (g >= 4) v = op(v, dpp<DPP_XOR2>(__float_as_uint(v)));
    if (g >= 8) v = op(v, dpp<DPP_HALF_MIRROR>(__float_as_uint(v)));
    if (g >= 16) v = op(v, dpp<DPP_ROW_MIRROR>(__float_as_uint(v)));
    if (g >= 32) v = op(v, (uint32_t)__shfl_xor((int)__float_as_uint(v), 16, 64));
    if (g >= 64) v = op(v, (uint32_t)__shfl_xor((int)__float_as_uint(v), 32, 64));
    return v;
}

// AMAX: the tensor pre-pass of NVFP4 scales instead: the finite maximum of
// |x| (after the rotation) per workgroup into p.amax_parts
// MODE (power-of-two scales, FP8S false): 0 E8M0 to nearest, 1 E8M0 with
// stochastic rounding, 2 E3M0 to nearest, 3 INT4 elements with E8M0 scales to
// nearest (plain or min/max).  Each has its own instantiation, so that the
// Philox state or the other modes' logic does not weigh on the rest.  PLAIN:
// no rotation and no macro scales, known at compile time, so that none of
// their code (or its branches) is in the loop.  DQ: with the dense dequantized
// output (its own instantiation, so the others keep their registers).
template <bool BF, bool FP8S, bool ST, bool AMAX = false, int MODE = 0, bool PLAIN = false, bool DQ = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DQ ? 2 : 4, 8))) void k_rows_hw(QParams p, HwArgs h) {
    const int hg = PLAIN ? 0 : h.hg, mg = PLAIN ? 0 : h.mg;
    constexpr int EPC = BF ? 8 : 4;        // elements per 16-byte chunk
    constexpr int CB = EPC / 2;            // code bytes per chunk
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (h.nchunks + TILE_CH - 1) / TILE_CH;
    const int64_t step = (int64_t)gridDim.x * (NT / 64);
    const char* xin = static_cast<const char*>(p.x);
    const int lin = lane * 16, lco = lane * CB;
    const bool lead = lane % h.g == 0;
    const int lsc = lead ? lane / h.g : OOB_OFFSET;
    const int lmc = (mg && lane % mg == 0) ? lane / mg : OOB_OFFSET;
    const int lof = lead ? (lane / h.g) * 2 : OOB_OFFSET;   // INT4 min/max: bf16 offset bytes
    const float gts = (FP8S && h.nvfp4 && !AMAX) ? *p.tensor_scale : 1.0f;
    const int eref = (!FP8S && !AMAX && MODE == 2) ? *p.ref_exp : 0;
    const float rgts = 1.0f / gts;
    // the statistics read zero dequantized values off the codes unless an NVFP4
    // tensor scale is small enough for a nonzero code's value to underflow to 0
    // (the smallest nonzero one is 0.5 x 2^-9 x g)
    const bool codes_decide = MODE != 3 && (!(FP8S && h.nvfp4) || gts >= 0x1p-100f);
    uint32_t tmax = 0;                     // AMAX: finite maximum of |x| as float bits
    double s2d = 0.0, e2d = 0.0;
    uint32_t nz = 0, fl = 0, zb = 0;
    // fp8 block scales: per scale code c the block scale s_b, the divisor S
    // (s_b times the NVFP4 tensor scale, rounded to fp32) and RN(1 / S), by the
    // same arithmetic the loop would spend on them per chunk, once per workgroup
    __shared__ f4v stab[(FP8S && !AMAX) ? 256 : 1];
    if constexpr (FP8S && !AMAX) {
        const int c = threadIdx.x;         // NT == 256 threads: one code each
        const float sbc = fp8_value(h.ue5 != 0, c);
        const float Sc = h.nvfp4 ? sbc * gts : sbc;
        stab[c] = f4v{sbc, Sc, 1.0f / Sc, 0.f};
        __syncthreads();
    }

    auto valid = [&](int64_t t) -> int {
        const int64_t r = h.nchunks - t * TILE_CH;
        return r <= 0 ? 0 : (r < TILE_CH ? (int)r : TILE_CH);
    };
    for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + wave; t < ntiles; t += step) {
        const int nv = valid(t);
        const rsrc_t rx = buf(xin + t * TILE_CH * 16, nv * 16);
        const rsrc_t rc = buf(p.codes + t * TILE_CH * CB, nv * CB);
        const rsrc_t rs = buf(p.scales + t * (TILE_CH / h.g), nv / h.g);
        const rsrc_t rm = buf(mg ? p.macro + t * (TILE_CH / (mg ? mg : 1)) : p.codes, mg ? nv / mg : 0);
        const rsrc_t ro = buf(MODE == 3 && h.asym ? (const void*)(p.offsets + t * (TILE_CH / h.g)) : (const void*)p.codes,
                              MODE == 3 && h.asym ? (nv / h.g) * 2 : 0);
        u32x4 w[FAST_NL];
#pragma unroll
        for (int k = 0; k < FAST_NL; k++)
            w[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, lin + k * 1024, 0, CPOL_NT));
#pragma unroll
        for (int k = 0; k < FAST_NL; k++) {
            float x[EPC];
#pragma unroll
            for (int i = 0; i < EPC; i++)
                x[i] = BF ? ((i & 1) ? bf16hi(w[k][i >> 1]) : bf16lo(w[k][i >> 1])) : __uint_as_float(w[k][i]);
            if (hg) {
#pragma unroll
                for (int span = 1; span < EPC; span <<= 1) {
#pragma unroll
                    for (int i = 0; i < EPC; i++) {
                        if (i & span) continue;
                        const float a = x[i], b = x[i + span];
                        x[i] = a + b;
                        x[i + span] = a - b;
                    }
                }
                if (hg > 1) had_stage<1>(x, lane);
                if (hg > 2) had_stage<2>(x, lane);
                if (hg > 4) had_stage<4>(x, lane);
                if (hg > 8) had_stage<8>(x, lane);
                if (hg > 16) had_stage<16>(x, lane);
#pragma unroll
                for (int i = 0; i < EPC; i++) x[i] = x[i] * h.hconst;
            }
            if constexpr (AMAX) {
#pragma unroll
                for (int i = 0; i < EPC; i++) {
                    const uint32_t u = __float_as_uint(x[i]) & 0x7fffffffu;
                    if (u < 0x7f800000u) tmax = max(tmax, u);
                }
                continue;
            }
            // macro-block scale over mg lanes
            float y[EPC];
            float sM = 1.0f;
            uint32_t smc = 0x38u;
            if (mg) {
                uint32_t mb = 0;
#pragma unroll
                for (int i = 0; i < EPC; i++) {
                    const uint32_t u = __float_as_uint(x[i]) & 0x7fffffffu;
                    if (u < 0x7f800000u) mb = max(mb, u);
                }
                mb = group_max_g(mb, mg);
                if (mb) {
                    const float tt = __uint_as_float(mb) / 6.0f;
                    const float mu = tt * pow2f(-flog2(tt));
                    smc = (uint32_t)fp8_code(false, mu);
                    sM = fp8_value(false, (int)smc);
                }
                if (wave_needs_exact_div(x)) {
#pragma unroll
                    for (int i = 0; i < EPC; i++) y[i] = x[i] / sM;
                } else {
                    const float rM = 1.0f / sM;
#pragma unroll
                    for (int i = 0; i < EPC; i++) y[i] = div_by(x[i], sM, rM);
                }
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)smc, rm, lmc + k * (64 / mg), 0, 0);
            } else {
#pragma unroll
                for (int i = 0; i < EPC; i++) y[i] = x[i];
            }
            // the block maximum: float bits of |y|; NaN and Inf sort above every finite value.
            // bf16 in, fp8 scales, no rotation (y is x): from the 15-bit magnitudes,
            // two per instruction, with the least nonzero magnitude minus one (zero
            // wraps to the top) for the exact-division guard
            const bool raw = BF && FP8S && hg == 0;
            u32x4 m4 = w[k] & 0x7fff7fffu;
            uint32_t am = 0, lo16 = 0xffffu;
            if (raw) {
                const us2 mx = __builtin_elementwise_max(__builtin_elementwise_max(as_us2(m4.x), as_us2(m4.y)),
                                                         __builtin_elementwise_max(as_us2(m4.z), as_us2(m4.w)));
                const us2 one = {1, 1};
                const us2 mn = __builtin_elementwise_min(
                    __builtin_elementwise_min(as_us2(m4.x) - one, as_us2(m4.y) - one),
                    __builtin_elementwise_min(as_us2(m4.z) - one, as_us2(m4.w) - one));
                am = max((uint32_t)mx[0], (uint32_t)mx[1]) << 16;
                lo16 = min((uint32_t)mn[0], (uint32_t)mn[1]);
            } else {
#pragma unroll
                for (int i = 0; i < EPC; i++) am = max(am, __float_as_uint(y[i]) & 0x7fffffffu);
            }
            am = group_max_g(am, h.g);
            const bool nonfinite = am >= 0x7f800000u;
            uint32_t cw = 0, code;
            float d[EPC];
            if constexpr (!FP8S) {
              if constexpr (MODE == 3) {
                // INT4, E8M0 scale 2^e, to nearest.  Min/max variant: offset o =
                // bf16 floor of the block minimum, e from the range max - o, codes
                // 0 .. 15 of (x - o) 2^-e (a negative value takes 0); plain: e
                // from max |x|, codes -7 .. 7 in two's complement.  The integer
                // nearest |v| ties to even and is capped at the largest code.
                const Elem E4 = make_elem(INT4, h.asym);
                float lo = y[0], hi = y[0];
#pragma unroll
                for (int i = 1; i < EPC; i++) { lo = fminf(lo, y[i]); hi = fmaxf(hi, y[i]); }
                int e;
                uint16_t ob = 0;
                float o = 0.f;
                if (h.asym) {
                    lo = group_fext_g<false>(lo, h.g);
                    hi = group_fext_g<true>(hi, h.g);
                    ob = bf16_floor(lo);
                    o = bf16f(ob);
                    const float R = hi - o;
                    e = R > 0.f ? e8m0_exp(p.rule, p.tau, E4, R) : -127;
                } else {
                    e = e8m0_exp(p.rule, p.tau, E4, __uint_as_float(am));
                }
                const float down = pow2f(-e), up = pow2f(e), qcap = (float)E4.maxidx;
                cw = 0;
#pragma unroll
                for (int i = 0; i < EPC; i++) {
                    const float v = (h.asym ? (y[i] - o) : y[i]) * down;
                    const bool neg = (__float_as_uint(v) >> 31) != 0;
                    const float m = (h.asym && neg) ? 0.f : fabsf(v);
                    const int idx = (int)fminf(rintf(m), qcap);
                    const int sv = (!h.asym && neg) ? -idx : idx;
                    cw |= (uint32_t)(h.asym ? idx : (sv & 0xf)) << (4 * i);
                    d[i] = (float)sv * up;
                    if (h.asym) d[i] = d[i] + o;
                }
                if (nonfinite) cw = 0;
                code = nonfinite ? 0xffu : (uint32_t)(e + 127);
                if (h.asym)
                    __builtin_amdgcn_raw_buffer_store_b16(nonfinite ? (uint16_t)0 : ob, ro, lof + k * (64 / h.g) * 2, 0, 0);
              } else if constexpr (MODE == 2) {
                // E3M0: step-down c = e_ref - e_ceil(amax, 6) clamped to 0 .. 7 (7
                // for an all-zero block), scale 2^(e_ref - c); the elements scaled,
                // rounded by the pair convert and decoded with 2^e as the general
                // row kernel does
                int cd = 7;
                if (am != 0u && !nonfinite) {
                    cd = eref - e_ceil(__uint_as_float(am), 6.0f);
                    cd = cd < 0 ? 0 : (cd > 7 ? 7 : cd);
                }
                const int e = eref - cd;
                const float down = pow2f(-e), up = pow2f(e);
                float v[EPC];
#pragma unroll
                for (int i = 0; i < EPC; i++) v[i] = y[i] * down;
                cw = enc_fp4<EPC / 2>(v, 1.0f);
                if (nonfinite) cw = 0;
                dec_fp4<EPC / 2>(cw, up, d);
                code = nonfinite ? 0xffu : (uint32_t)cd;
              } else {
                uint32_t sbits;
                if (h.floor_rule) sbits = __builtin_elementwise_sub_sat(am & 0x7f800000u, 0x01000000u);
                else sbits = (uint32_t)(fast_exp<false>(am, h.lq, h.fq) + 127) << 23;
                code = sbits >> 23;
                const float scale = __uint_as_float(sbits);
                if constexpr (MODE == 1) {
                    // stochastic rounding of y 2^-e (e = code - 127, the general
                    // kernel's single rounding): the draws of the chunk's elements,
                    // 8 per Philox call at their linear indices (rows are dense)
                    const uint64_t ch = (uint64_t)(t * TILE_CH + k * 64 + lane);
                    uint32_t r[8];
                    draws8(p.seed, p.off, BF ? ch : (ch >> 1), r);
                    const float down = pow2f(127 - (int)code);
                    cw = 0;
#pragma unroll
                    for (int i = 0; i < EPC; i++)
                        cw |= (uint32_t)sr_e2m1(y[i] * down, BF ? r[i] : r[4 * (int)(ch & 1) + i]) << (4 * i);
                } else {
                    cw = enc_fp4<EPC / 2>(y, scale);
                }
                if (nonfinite) cw = 0;
                dec_fp4<EPC / 2>(cw, scale, d);
                if (mg) {
#pragma unroll
                    for (int i = 0; i < EPC; i++) d[i] = d[i] * sM;
                }
                if (nonfinite) code = 0xffu;
              }
            } else {
                // RN(1/6) = 0x3e2aaaab
                float tt = div_lane(__uint_as_float(am), 6.0f, __uint_as_float(0x3e2aaaabu));
                if (h.nvfp4) tt = div_lane(tt, gts, rgts);
                const int sc = fp8_code(h.ue5 != 0, tt);
                const f4v te = stab[sc];
                const float sb = te[0], S = te[1];
                float v[EPC];
                // a nonzero magnitude below 2^-96 (bf16 0x0f80) or a non-finite one
                // in any lane: the exact division
                const bool exact = raw ? __any(lo16 < 0x0f7fu || am >= 0x7f800000u) : wave_needs_exact_div(y);
                if (exact) {
#pragma unroll
                    for (int i = 0; i < EPC; i++) v[i] = y[i] / S;
                } else {
                    const float rS = te[2];
#pragma unroll
                    for (int i = 0; i < EPC; i++) v[i] = div_by(y[i], S, rS);
                }
                if (__any(S == 0.f)) {
#pragma unroll
                    for (int i = 0; i < EPC; i++)
                        if (S == 0.f) v[i] = (__float_as_uint(y[i]) >> 31) ? -0.f : 0.f;
                }
                cw = enc_fp4<EPC / 2>(v, 1.0f);
                if (nonfinite) cw = 0;
                dec_fp4<EPC / 2>(cw, 1.0f, d);
#pragma unroll
                for (int i = 0; i < EPC; i++) {
                    d[i] = d[i] * sb;
                    if (h.nvfp4) d[i] = d[i] * gts;
                }
                code = nonfinite ? (h.ue5 ? 0xffu : 0x7fu) : (uint32_t)sc;
            }
            if (__any(nonfinite)) {
#pragma unroll
                for (int i = 0; i < EPC; i++)
                    if (nonfinite) d[i] = __uint_as_float(0x7fc00000u);
            }
            if constexpr (DQ) {
                // the dequantized values, dense: fp32, or bf16 rounded to nearest even
                const int dqb = p.dq_bf16 ? 2 : 4;
                const rsrc_t rdq = buf(static_cast<char*>(p.dq) + t * TILE_CH * EPC * dqb, nv * EPC * dqb);
                if (p.dq_bf16) {
                    uint32_t b[EPC / 2];
#pragma unroll
                    for (int j = 0; j < EPC / 2; j++) b[j] = bf16_rne(d[2 * j]) | ((uint32_t)bf16_rne(d[2 * j + 1]) << 16);
                    if constexpr (BF)
                        __builtin_amdgcn_raw_buffer_store_b128((u32x4){b[0], b[1], b[2], b[3]}, rdq, lane * 16 + k * 1024, 0,
                                                               0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b64((u32x2){b[0], b[1]}, rdq, lane * 8 + k * 512, 0, 0);
                } else {
                    const u32x4 o0 = {__float_as_uint(d[0]), __float_as_uint(d[1]), __float_as_uint(d[2]),
                                      __float_as_uint(d[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(o0, rdq, lane * (EPC * 4) + k * 64 * (EPC * 4), 0, 0);
                    if constexpr (BF) {
                        const u32x4 o1 = {__float_as_uint(d[4]), __float_as_uint(d[5]), __float_as_uint(d[6]),
                                          __float_as_uint(d[7])};
                        __builtin_amdgcn_raw_buffer_store_b128(o1, rdq, lane * 32 + 16 + k * 64 * 32, 0, 0);
                    }
                }
            }
            if constexpr (BF) __builtin_amdgcn_raw_buffer_store_b32(cw, rc, lco + k * 64 * CB, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b16((uint16_t)cw, rc, lco + k * 64 * CB, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, rs, lsc + k * (64 / h.g), 0, 0);
            if constexpr (ST) {
                float s2c = 0.f, e2c = 0.f;
                uint32_t nzl = 0, zin = 0;
                if (raw) {
                    // x is the bf16 input: x^2 by pairs, and the zero inputs from the
                    // magnitudes (adding 0x7fff sets bit 15 of a nonzero one)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        s2c = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w[k][j]), as_bf2(w[k][j]), s2c, false);
                    const uint32_t g01 = __builtin_amdgcn_perm(m4.x + 0x7fff7fffu, m4.y + 0x7fff7fffu, 0x07050301u);
                    const uint32_t g23 = __builtin_amdgcn_perm(m4.z + 0x7fff7fffu, m4.w + 0x7fff7fffu, 0x07050301u);
                    zin = EPC - (__builtin_popcount(g01 & 0x80808080u) + __builtin_popcount(g23 & 0x80808080u));
#pragma unroll
                    for (int i = 0; i < EPC; i++) {
                        const float ri = x[i] - d[i];
                        e2c = __builtin_fmaf(ri, ri, e2c);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < EPC; i++) {
                        const float ri = x[i] - d[i];
                        s2c = __builtin_fmaf(x[i], x[i], s2c);
                        e2c = __builtin_fmaf(ri, ri, e2c);
                        zin += (x[i] == 0.f) ? 1u : 0u;
                    }
                }
                nz += EPC - zin;                       // NaN counts as non-zero
                if (codes_decide) {
                    // a dequantized value is zero exactly when its code's magnitude
                    // is, and a zero input always gets such a code: flushed = zero
                    // codes - zero inputs; a non-finite block (d NaN) flushes nothing
                    // and is not all zero
                    const uint32_t tm = cw & (BF ? 0x77777777u : 0x7777u);
                    const uint32_t zc = __builtin_popcount(~(tm + (BF ? 0x77777777u : 0x7777u)) &
                                                           (BF ? 0x88888888u : 0x8888u));
                    fl += nonfinite ? 0u : zc - zin;
                    nzl = (nonfinite || tm != 0u) ? 1u : 0u;
                } else {
#pragma unroll
                    for (int i = 0; i < EPC; i++) {
                        fl += (x[i] != 0.f && d[i] == 0.f);
                        nzl |= (d[i] != 0.f) ? 1u : 0u;
                    }
                }
                if (fabsf(s2c) < INFINITY && fabsf(e2c) < INFINITY) {
                    s2d += (double)s2c;
                    e2d += (double)e2c;
                } else {
#pragma unroll
                    for (int i = 0; i < EPC; i++) {
                        const double xd = x[i], dd = d[i];
                        s2d += xd * xd;
                        e2d += (xd - dd) * (xd - dd);
                    }
                }
                nzl = group_max_g(nzl, h.g);
                zb += (lead && nzl == 0 && lane + k * 64 < nv) ? 1u : 0u;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (AMAX) {
        const float a = block_max<NT>(__uint_as_float(tmax));
        if (threadIdx.x == 0) p.amax_parts[blockIdx.x] = a;
    } else if constexpr (ST) {
        block_stats<NT>(s2d, e2d, nz, fl, zb, p.parts + blockIdx.x);
    }
}

int fast_g(const QParams& p) { return p.bc / (p.in_bf16 ? 8 : 4); }

int64_t fast_groups(const QParams& p) {
    const int64_t nchunks = p.rows * p.cols / (p.in_bf16 ? 8 : 4);
    const int64_t ntiles = (nchunks + TILE_CH - 1) / TILE_CH;
    return (ntiles + NT / 64 - 1) / (NT / 64);
}

// workgroups the device keeps resident at once for kernel `k`, on the current
// device; the caller keeps one cache per kernel
template <typename K>
int64_t resident(K k, int64_t* cache) {
    int64_t v = __atomic_load_n(cache, __ATOMIC_RELAXED);
    if (v) return v;
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, NT, 0) != hipSuccess || cus <= 0 || per <= 0)
        return FAST_MAX_GRID;
    v = (int64_t)cus * per;
    __atomic_store_n(cache, v, __ATOMIC_RELAXED);
    return v;
}

template <bool BF, int G, bool FLOOR, bool ST, bool DQ>
hipError_t launch_fast(const QParams& p, hipStream_t s, int64_t* grid) {
    auto k = k_rows_fast<BF, G, FLOOR, ST, DQ>;
    static int64_t cache = 0;   // one per instantiation
    int64_t g = fast_groups(p);
    const int64_t r = resident(k, &cache);
    if (g > r) g = r;
    if (g > FAST_MAX_GRID) g = FAST_MAX_GRID;
    *grid = g;
    if (g == 0) return hipSuccess;
    // CEIL is OAS with tau = 6, E2M1's largest magnitude
    float q = p.rule == RULE_OAS ? p.tau : 6.0f;
    uint32_t qb;
    memcpy(&qb, &q, 4);
    const int lq = (int)(qb >> 23) - 127;
    const uint32_t fq = qb & 0x7fffffu;
    const int64_t nchunks = p.rows * p.cols / (BF ? 8 : 4);
    k<<<g, NT, 0, s>>>(p, nchunks, lq, fq);
    return hipGetLastError();
}

template <bool BF, int G, bool DQ>
hipError_t launch_fast_d(const QParams& p, hipStream_t s, int64_t* grid) {
    const bool st = p.parts != nullptr;
    if (p.rule == RULE_FLOOR)
        return st ? launch_fast<BF, G, true, true, DQ>(p, s, grid) : launch_fast<BF, G, true, false, DQ>(p, s, grid);
    return st ? launch_fast<BF, G, false, true, DQ>(p, s, grid) : launch_fast<BF, G, false, false, DQ>(p, s, grid);
}

template <bool BF, int G>
hipError_t launch_fast_g(const QParams& p, hipStream_t s, int64_t* grid) {
    return p.dq ? launch_fast_d<BF, G, true>(p, s, grid) : launch_fast_d<BF, G, false>(p, s, grid);
}

}  // namespace

bool rows_fast_ok(const QParams& p) {
    const int g = fast_g(p);
    return p.elem == E2M1 && p.scale == SC_E8M0 && p.round == RTNE && !p.asym && !p.had && !p.macro_cols &&
           p.br == 1 && p.ld == p.cols && g * (p.in_bf16 ? 8 : 4) == p.bc && g >= 1 && g <= 64 &&
           (g & (g - 1)) == 0 && p.cols % p.bc == 0;
}

int64_t rows_fast_grid(const QParams& p) {
    const int64_t g = fast_groups(p);
    return g < FAST_MAX_GRID ? g : FAST_MAX_GRID;
}

hipError_t launch_rows_fast(const QParams& p, hipStream_t s, int64_t* grid) {
    *grid = 0;
    const int g = fast_g(p);
#define MX_FAST_CASE(BFv, Gv) \
    if (p.in_bf16 == (BFv) && g == (Gv)) return launch_fast_g<BFv, Gv>(p, s, grid);
    MX_FAST_CASE(true, 1) MX_FAST_CASE(true, 2) MX_FAST_CASE(true, 4) MX_FAST_CASE(true, 8) MX_FAST_CASE(true, 16)
    MX_FAST_CASE(true, 32) MX_FAST_CASE(false, 2) MX_FAST_CASE(false, 4) MX_FAST_CASE(false, 8)
    MX_FAST_CASE(false, 16) MX_FAST_CASE(false, 32) MX_FAST_CASE(false, 64)
#undef MX_FAST_CASE
    return hipErrorInvalidValue;
}

namespace {
template <bool BF, int G, bool FLOOR, bool ST>
hipError_t launch_fast_many(const QParams& p, FastMany& m, hipStream_t s, int64_t* grid) {
    auto k = k_rows_fast_many<BF, G, FLOOR, ST>;
    static int64_t cache = 0;   // one per instantiation
    int64_t cap = resident(k, &cache);
    if (cap > FAST_MAX_GRID) cap = FAST_MAX_GRID;
    // the resident workgroups shared in proportion to the jobs' chunks (so the
    // waves of every job walk about the same number of tiles), at least one
    // and at most as many as a job's tiles fill; never more than fit at once
    int64_t total = 0;
    for (int i = 0; i < m.count; i++) total += m.job[i].nchunks;
    const int64_t share = cap > m.count ? cap - m.count : 1;
    int64_t b0 = 0;
    for (int i = 0; i < m.count; i++) {
        FastJob& J = m.job[i];
        const int64_t ntiles = (J.nchunks + TILE_CH - 1) / TILE_CH;
        const int64_t groups = (ntiles + NT / 64 - 1) / (NT / 64);
        int64_t nb = (int64_t)((double)share * (double)J.nchunks / (double)total);
        nb = std::min(std::max(nb, (int64_t)1), groups);
        J.b0 = b0;
        J.nb = nb;
        b0 += nb;
    }
    *grid = b0;
    if (b0 == 0) return hipSuccess;
    float q = p.rule == RULE_OAS ? p.tau : 6.0f;
    uint32_t qb;
    memcpy(&qb, &q, 4);
    k<<<b0, NT, 0, s>>>(m, (int)(qb >> 23) - 127, qb & 0x7fffffu);
    return hipGetLastError();
}

template <bool BF, int G>
hipError_t launch_fast_many_g(const QParams& p, FastMany& m, hipStream_t s, int64_t* grid) {
    const bool st = p.parts != nullptr;
    if (p.rule == RULE_FLOOR)
        return st ? launch_fast_many<BF, G, true, true>(p, m, s, grid) : launch_fast_many<BF, G, true, false>(p, m, s, grid);
    return st ? launch_fast_many<BF, G, false, true>(p, m, s, grid) : launch_fast_many<BF, G, false, false>(p, m, s, grid);
}
}  // namespace

bool rows_fp8_ok(const QParams& p) {
    return (p.elem == E4M3 || p.elem == E5M2) && p.scale == SC_E8M0 && p.round == RTNE && !p.asym && !p.had &&
           !p.macro_cols && p.br == 1 && p.bc == 32 && p.ld == p.cols && p.cols % 32 == 0;
}

namespace {
template <bool BF, bool ST, bool E5>
hipError_t launch_fp8_t(const QParams& p, hipStream_t s, int64_t* grid) {
    constexpr int G = BF ? 4 : 8;         // lanes per 32-element block
    auto k = k_rows_fp8<BF, G, ST, E5>;
    static int64_t cache = 0;   // one per instantiation
    int64_t g = fast_groups(p);
    const int64_t r = resident(k, &cache);
    if (g > r) g = r;
    if (g > FAST_MAX_GRID) g = FAST_MAX_GRID;
    *grid = g;
    if (g == 0) return hipSuccess;
    // CEIL is OAS with tau = Qmax, the format's largest magnitude
    const float q = p.rule == RULE_OAS ? p.tau : (E5 ? 57344.0f : 448.0f);
    uint32_t qb;
    memcpy(&qb, &q, 4);
    const int64_t nchunks = p.rows * p.cols / (BF ? 8 : 4);
    k<<<g, NT, 0, s>>>(p, nchunks, (int)(qb >> 23) - 127, qb & 0x7fffffu, p.rule == RULE_FLOOR ? 1 : 0);
    return hipGetLastError();
}
}  // namespace

int64_t rows_fp8_grid(const QParams& p) { return rows_fast_grid(p); }

hipError_t launch_rows_fp8(const QParams& p, hipStream_t s, int64_t* grid) {
    *grid = 0;
    const bool st = p.parts != nullptr, e5 = p.elem == E5M2;
    if (p.in_bf16) {
        if (e5) return st ? launch_fp8_t<true, true, true>(p, s, grid) : launch_fp8_t<true, false, true>(p, s, grid);
        return st ? launch_fp8_t<true, true, false>(p, s, grid) : launch_fp8_t<true, false, false>(p, s, grid);
    }
    if (e5) return st ? launch_fp8_t<false, true, true>(p, s, grid) : launch_fp8_t<false, false, true>(p, s, grid);
    return st ? launch_fp8_t<false, true, false>(p, s, grid) : launch_fp8_t<false, false, false>(p, s, grid);
}

bool rows_fp6_ok(const QParams& p) {
    return (p.elem == E2M3 || p.elem == E3M2) && p.scale == SC_E8M0 && p.round == RTNE && !p.asym && !p.had &&
           !p.macro_cols && p.br == 1 && p.bc == 32 && p.ld == p.cols && p.cols % 32 == 0;
}

int64_t rows_fp6_grid(const QParams& p) {
    const int64_t tiles = (p.rows * p.cols + FP6_TILE - 1) / FP6_TILE;
    const int64_t g = (tiles + NT / 64 - 1) / (NT / 64);
    return g < FAST_MAX_GRID ? g : FAST_MAX_GRID;
}

namespace {
template <bool BF, bool ST, bool E3>
hipError_t launch_fp6_t(const QParams& p, hipStream_t s, int64_t* grid) {
    auto k = k_rows_fp6<BF, ST, E3>;
    static int64_t cache = 0;   // one per instantiation
    int64_t g = rows_fp6_grid(p);
    const int64_t r = resident(k, &cache);
    if (g > r) g = r;
    *grid = g;
    if (g == 0) return hipSuccess;
    // CEIL is OAS with tau = Qmax, the format's largest magnitude
    const float q = p.rule == RULE_OAS ? p.tau : (E3 ? 28.0f : 7.5f);
    uint32_t qb;
    memcpy(&qb, &q, 4);
    k<<<g, NT, 0, s>>>(p, p.rows * p.cols, (int)(qb >> 23) - 127, qb & 0x7fffffu, p.rule == RULE_FLOOR ? 1 : 0);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_rows_fp6(const QParams& p, hipStream_t s, int64_t* grid) {
    *grid = 0;
    const bool st = p.parts != nullptr, e3 = p.elem == E3M2;
    if (p.in_bf16) {
        if (e3) return st ? launch_fp6_t<true, true, true>(p, s, grid) : launch_fp6_t<true, false, true>(p, s, grid);
        return st ? launch_fp6_t<true, true, false>(p, s, grid) : launch_fp6_t<true, false, false>(p, s, grid);
    }
    if (e3) return st ? launch_fp6_t<false, true, true>(p, s, grid) : launch_fp6_t<false, false, true>(p, s, grid);
    return st ? launch_fp6_t<false, true, false>(p, s, grid) : launch_fp6_t<false, false, false>(p, s, grid);
}

hipError_t launch_rows_fast_many(const QParams& p, FastMany& m, hipStream_t s, int64_t* grid) {
    *grid = 0;
    if (m.count < 1 || m.count > MANY_MAX) return hipErrorInvalidValue;
    const int g = fast_g(p);
#define MX_FAST_CASE(BFv, Gv) \
    if (p.in_bf16 == (BFv) && g == (Gv)) return launch_fast_many_g<BFv, Gv>(p, m, s, grid);
    MX_FAST_CASE(true, 1) MX_FAST_CASE(true, 2) MX_FAST_CASE(true, 4) MX_FAST_CASE(true, 8) MX_FAST_CASE(true, 16)
    MX_FAST_CASE(true, 32) MX_FAST_CASE(false, 2) MX_FAST_CASE(false, 4) MX_FAST_CASE(false, 8)
    MX_FAST_CASE(false, 16) MX_FAST_CASE(false, 32) MX_FAST_CASE(false, 64)
#undef MX_FAST_CASE
    return hipErrorInvalidValue;
}

namespace {
typedef void (*HwKernel)(QParams, HwArgs);

// the instantiation for a mode, with or without rotation and macro scales
// (E8M0 to nearest with neither takes the MXFP4 kernel, so it has no plain
// one), with or without the dequantized output
template <bool BF, bool FP8S, bool ST, int MODE, bool DQ>
HwKernel hw_kernel_d(bool plain) {
    if constexpr (FP8S || MODE != 0)
        if (plain) return k_rows_hw<BF, FP8S, ST, false, MODE, true, DQ>;
    return k_rows_hw<BF, FP8S, ST, false, MODE, false, DQ>;
}

template <bool BF, bool FP8S, bool ST, int MODE>
HwKernel hw_kernel(bool plain, bool dq) {
    return dq ? hw_kernel_d<BF, FP8S, ST, MODE, true>(plain) : hw_kernel_d<BF, FP8S, ST, MODE, false>(plain);
}

template <bool BF, bool FP8S>
hipError_t launch_hw_t(const QParams& p, const HwArgs& h, hipStream_t s, int64_t* grid) {
    const bool st = p.parts != nullptr;
    const bool plain = h.hg == 0 && h.mg == 0;
    const bool dq = p.dq != nullptr;
    constexpr int M1 = FP8S ? 0 : 1, M2 = FP8S ? 0 : 2, M3 = FP8S ? 0 : 3;
    const int mode = FP8S ? 0 : (h.int4 ? 3 : (h.sr ? 1 : (h.e3m0 ? 2 : 0)));
    const HwKernel k =
        mode == 1   ? (st ? hw_kernel<BF, FP8S, true, M1>(plain, dq) : hw_kernel<BF, FP8S, false, M1>(plain, dq))
        : mode == 2 ? (st ? hw_kernel<BF, FP8S, true, M2>(plain, dq) : hw_kernel<BF, FP8S, false, M2>(plain, dq))
        : mode == 3 ? (st ? hw_kernel<BF, FP8S, true, M3>(plain, dq) : hw_kernel<BF, FP8S, false, M3>(plain, dq))
                    : (st ? hw_kernel<BF, FP8S, true, 0>(plain, dq) : hw_kernel<BF, FP8S, false, 0>(plain, dq));
    // one per statistics, mode, plain and dequant variant
    static int64_t cache[32] = {};
    int64_t g = fast_groups(p);
    const int64_t r = resident(k, &cache[(st ? 1 : 0) + 2 * mode + (plain ? 8 : 0) + (dq ? 16 : 0)]);
    if (g > r) g = r;
    if (g > FAST_MAX_GRID) g = FAST_MAX_GRID;
    *grid = g;
    if (g == 0) return hipSuccess;
    k<<<g, NT, 0, s>>>(p, h);
    return hipGetLastError();
}
}  // namespace

namespace {
void hw_args(const QParams& p, HwArgs& h) {
    const int epc = p.in_bf16 ? 8 : 4;
    h.nchunks = p.rows * p.cols / epc;
    h.g = p.bc / epc;
    h.hg = p.had ? p.had / epc : 0;
    h.mg = p.macro_cols ? 128 / epc : 0;
    h.floor_rule = p.rule == RULE_FLOOR;
    const float q = p.rule == RULE_OAS ? p.tau : 6.0f;
    uint32_t qb;
    memcpy(&qb, &q, 4);
    h.lq = (int)(qb >> 23) - 127;
    h.fq = qb & 0x7fffffu;
    h.ue5 = p.scale == SC_UE5M3;
    h.nvfp4 = p.scale == SC_NVFP4;
    h.sr = p.round == SR;
    h.e3m0 = p.scale == SC_E3M0;
    h.int4 = p.elem == INT4;
    h.asym = p.asym;
    const uint32_t hc = p.had == 16 ? 0x3E800000u : p.had == 32 ? 0x3E3504F3u : p.had == 64 ? 0x3E000000u : 0x3DB504F3u;
    memcpy(&h.hconst, &hc, 4);
}
}  // namespace

bool rows_hw_ok(const QParams& p) {
    const int epc = p.in_bf16 ? 8 : 4;
    const bool scale_ok = p.scale == SC_E8M0 || p.scale == SC_UE4M3 || p.scale == SC_UE5M3 || p.scale == SC_NVFP4 ||
                          p.scale == SC_E3M0;
    const int g = p.bc / epc;
    const bool round_ok = p.round == RTNE || (p.round == SR && p.scale == SC_E8M0);
    const bool elem_ok = (p.elem == E2M1 && !p.asym) ||
                         (p.elem == INT4 && p.round == RTNE && p.scale == SC_E8M0 && !p.macro_cols);
    return elem_ok && round_ok && p.br == 1 && p.ld == p.cols && scale_ok &&
           g >= 1 && g <= 64 && g * epc == p.bc && (!p.had || p.had >= epc) && (!p.macro_cols || p.scale == SC_E8M0);
}

int64_t rows_hw_grid(const QParams& p) { return rows_fast_grid(p); }

hipError_t launch_rows_hw(const QParams& p, hipStream_t s, int64_t* grid) {
    *grid = 0;
    HwArgs h;
    hw_args(p, h);
    const bool fp8s = p.scale == SC_UE4M3 || p.scale == SC_UE5M3 || p.scale == SC_NVFP4;
    if (p.in_bf16) return fp8s ? launch_hw_t<true, true>(p, h, s, grid) : launch_hw_t<true, false>(p, h, s, grid);
    return fp8s ? launch_hw_t<false, true>(p, h, s, grid) : launch_hw_t<false, false>(p, h, s, grid);
}

// The NVFP4 / E3M0 tensor pre-pass (the finite maximum of |x|, after the
// rotation when there is one): on the wave-tile kernel for a dense tensor of
// whole 16-byte chunks per row (rotated only in the row formats it takes),
// else on the general row kernel.  *grid: the partials written.
hipError_t launch_amax(const QParams& p, hipStream_t s, int64_t* grid) {
    QParams a = p;
    a.dq = nullptr;
    const int epc = a.in_bf16 ? 8 : 4;
    if (a.ld == a.cols && a.cols % epc == 0 && (!a.had || rows_hw_ok(a))) {
        HwArgs h;
        hw_args(a, h);
        if (h.g < 1) h.g = 1;   // the scale-block lanes are not used by the pre-pass
        auto k = a.in_bf16 ? k_rows_hw<true, true, false, true> : k_rows_hw<false, true, false, true>;
        static int64_t cache[2] = {0, 0};
        int64_t g = fast_groups(a);
        const int64_t r = resident(k, &cache[a.in_bf16 ? 1 : 0]);
        if (g > r) g = r;
        if (g > FAST_MAX_GRID) g = FAST_MAX_GRID;
        *grid = g;
        if (g == 0) return hipSuccess;
        k<<<g, NT, 0, s>>>(a, h);
        return hipGetLastError();
    }
    *grid = rows_grid(p);
    return launch_rows(p, true, s);
}

}  // namespace mxk
