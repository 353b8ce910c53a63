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
    if (bits == 4) {
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
                ob = bf16_rne((mx + mn) * 0.5f);
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
                c = encode(E, kind == 2 ? RTNE : p.round, v, rnd[k]);
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
        store_codes(p.codes + r * (E.bits == 4 ? p.cols / 2 : p.cols * 3 / 4), E.bits, c0, code, CH);
        if (p.dq) store_dq<CH>(p, r, c0, d);
    }
    if (p.parts) {
        double s2 = 0, e2 = 0;
        unsigned long long nz = 0, fl = 0;
        if (active) {
#pragma unroll
            for (int i = 0; i < CH; i++) {
                double xv = x[i], dv = d[i];
                s2 += xv * xv;
                e2 += (xv - dv) * (xv - dv);
                nz += (x[i] != 0.f);
                fl += (x[i] != 0.f && d[i] == 0.f);
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

int64_t amax_grid(const QParams& p) { return rows_grid(p); }


namespace {

// ---------------------------------------------------------------------------
// MXFP4 fast path: E2M1 elements, E8M0 scales (any exponent rule), round to
// nearest even, dense rows (ld == cols).  gfx950's V_CVT_SCALEF32_PK_FP4_*
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

template <bool BF, int G, bool FLOOR, bool ST>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G >= 32 ? 4 : (FLOOR ? (ST ? 8 : FAST_WAVES) : FAST_WAVES - 1), 8))) void k_rows_fast(QParams p, int64_t nchunks, int lq, uint32_t fq) {
    constexpr int EPC = BF ? 8 : 4;        // elements per chunk
    constexpr int CB = EPC / 2;            // code bytes per chunk
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (nchunks + TILE_CH - 1) / TILE_CH;
    const int64_t step = (int64_t)gridDim.x * (NT / 64);
    const char* xin = static_cast<const char*>(p.x);
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
        const rsrc_t rc = buf(p.codes + t * TILE_CH * CB, nv * CB);
        const rsrc_t rs = buf(p.scales + t * (TILE_CH / G), nv / G);
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

            if constexpr (ST) {
                // dequantized values straight from the codes (value * 2^e)
                float d[EPC];
                f2v dd[EPC / 2];
                dd[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 0);
                dd[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 1);
                if constexpr (BF) {
                    dd[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 2);
                    dd[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, scale, 3);
                }
#pragma unroll
                for (int j = 0; j < EPC / 2; j++) { d[2 * j] = dd[j][0]; d[2 * j + 1] = dd[j][1]; }
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
        for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + wave; t < ntiles; t += step) {
            u32x4 w1[FAST_NL];
            load(w1, t);
            work(w1, t);
        }
    } else {
        // two register tiles in ping-pong: one is worked on while the other loads
        int64_t t = (int64_t)blockIdx.x * (NT / 64) + wave;
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
    if constexpr (ST) block_stats<NT>(s2d, e2d, nz, fl, zb, p.parts + blockIdx.x);
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

template <bool BF, int G, bool FLOOR, bool ST>
hipError_t launch_fast(const QParams& p, hipStream_t s, int64_t* grid) {
    auto k = k_rows_fast<BF, G, FLOOR, ST>;
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

template <bool BF, int G>
hipError_t launch_fast_g(const QParams& p, hipStream_t s, int64_t* grid) {
    const bool st = p.parts != nullptr;
    if (p.rule == RULE_FLOOR)
        return st ? launch_fast<BF, G, true, true>(p, s, grid) : launch_fast<BF, G, true, false>(p, s, grid);
    return st ? launch_fast<BF, G, false, true>(p, s, grid) : launch_fast<BF, G, false, false>(p, s, grid);
}

}  // namespace

bool rows_fast_ok(const QParams& p) {
    const int g = fast_g(p);
    return p.elem == E2M1 && p.scale == SC_E8M0 && p.round == RTNE && !p.asym && !p.had && !p.macro_cols &&
           !p.dq && p.br == 1 && p.ld == p.cols && g * (p.in_bf16 ? 8 : 4) == p.bc && g >= 1 && g <= 64 &&
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

hipError_t launch_amax(const QParams& p, hipStream_t s) { return launch_rows(p, true, s); }

}  // namespace mxk
