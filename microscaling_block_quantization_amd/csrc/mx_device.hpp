// mx_device.hpp -- device helpers for the gfx950 microscaling kernels.
//
// Element encoders work on the fp32 bit pattern: a magnitude in the normal
// range of a minifloat is rounded to MB mantissa bits by an integer add with
// round-to-nearest-even carry, and the subnormal range by rintf of an exact
// power-of-two multiple.  Scale rules use exponent / significand comparisons
// on the bits.  Element grids and scale formats are those of the pages:
// E2M1 + E8M0 (MXFP4) and E2M1 + E4M3 + fp32 per-tensor scale (NVFP4),
// "Unveiling the Potential of Quantization with MXFP4", Sec. 2; UE5M3, "Is
// Finer Better?", technical summary; INT4 / E3M0 and the rounding modes, the
// ARITH 2025 MX-training report, main results.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxd {

enum { E2M1 = 0, INT4 = 1, E2M3 = 2, E3M2 = 3, E3M0 = 4, E4M3 = 5, E5M2 = 6 };
enum { SC_E8M0 = 0, SC_UE4M3 = 1, SC_NVFP4 = 2, SC_UE5M3 = 3, SC_E3M0 = 4 };
enum { RULE_FLOOR = 0, RULE_CEIL = 1, RULE_OAS = 2 };
enum { RTNE = 0, SR = 1, CEILR = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: non-temporal hint)
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

// 2^k as an exact fp32 for k in [-149, 127]
__device__ __forceinline__ float pow2f(int k) {
    return k >= -126 ? bitsf((uint32_t)(k + 127) << 23) : bitsf(1u << (k + 149));
}

// floor(log2 a) for finite a > 0
__device__ __forceinline__ int flog2(float a) {
    uint32_t u = fbits(a) & 0x7fffffffu;
    int be = (int)(u >> 23);
    if (be) return be - 127;
    return -149 + (31 - __clz(u));
}

// significand bits below the leading one, left-aligned to 23 bits
__device__ __forceinline__ uint32_t frac23(float a) {
    uint32_t u = fbits(a) & 0x7fffffffu;
    if (u >> 23) return u & 0x7fffffu;
    return (u << (__clz(u) - 8)) & 0x7fffffu;
}

// smallest e with Q * 2^e >= a   (a > 0 finite, Q > 0 normal)
__device__ __forceinline__ int e_ceil(float a, float Q) {
    int p = flog2(a) - flog2(Q);
    return frac23(a) <= frac23(Q) ? p : p + 1;
}

// ---- element formats -------------------------------------------------------
struct Elem {
    int kind;       // E2M1 ... E3M0
    int asym;       // INT4 min/max variant
    int bits;       // 4, 6 or 8
    float qmax;     // largest magnitude
    int emax;       // floor(log2(qmax))
    int maxidx;     // largest magnitude index
};

__host__ __device__ inline Elem make_elem(int kind, int asym) {
    Elem e;
    e.kind = kind;
    e.asym = asym;
    e.bits = (kind == E2M3 || kind == E3M2) ? 6 : (kind == E4M3 || kind == E5M2) ? 8 : 4;
    switch (kind) {
    case E2M1: e.qmax = 6.f; e.emax = 2; e.maxidx = 7; break;
    case INT4: e.qmax = asym ? 15.f : 7.f; e.emax = asym ? 3 : 2; e.maxidx = asym ? 15 : 7; break;
    case E2M3: e.qmax = 7.5f; e.emax = 2; e.maxidx = 31; break;
    case E3M2: e.qmax = 28.f; e.emax = 4; e.maxidx = 31; break;
    // FP8 (OCP): E4M3 magnitude 0x7F is NaN, E5M2 0x7C is Inf; both saturate
    case E4M3: e.qmax = 448.f; e.emax = 8; e.maxidx = 0x7e; break;
    case E5M2: e.qmax = 57344.f; e.emax = 15; e.maxidx = 0x7b; break;
    default: e.qmax = 16.f; e.emax = 4; e.maxidx = 7; break;  // E3M0
    }
    return e;
}

// minifloat with MB mantissa bits and exponent bias BIAS: nearest index (RNE)
// or the index of the largest grid value <= m (floor), for finite m >= 0 or +inf
template <int MB, int BIAS>
__device__ __forceinline__ int mf_index(float m, bool nearest) {
    constexpr int SH = 23 - MB;
    if (m < bitsf((uint32_t)(128 - BIAS) << 23)) {           // below 2^(1-BIAS)
        float s = m * bitsf((uint32_t)(127 + BIAS + MB - 1) << 23);
        return (int)(nearest ? rintf(s) : floorf(s));
    }
    uint32_t u = fbits(m);
    if (nearest) u += ((1u << (SH - 1)) - 1u) + ((u >> SH) & 1u);
    uint32_t hi = u >> SH;
    return (int)(hi - ((uint32_t)(127 - BIAS) << MB));
}

template <int MB, int BIAS>
__device__ __forceinline__ float mf_value(int idx) {
    if (idx < (1 << MB)) return (float)idx * bitsf((uint32_t)(128 - BIAS - MB) << 23);
    return bitsf((uint32_t)(idx + ((127 - BIAS) << MB)) << (23 - MB));
}

// index of the magnitude grid for m >= 0: nearest-even (nearest) or floor
__device__ __forceinline__ int grid_index(const Elem& E, float m, bool nearest) {
    int i;
    switch (E.kind) {
    case E2M1: i = mf_index<1, 1>(m, nearest); break;
    case E2M3: i = mf_index<3, 1>(m, nearest); break;
    case E3M2: i = mf_index<2, 3>(m, nearest); break;
    case E4M3: i = mf_index<3, 7>(m, nearest); break;
    case E5M2: i = mf_index<2, 15>(m, nearest); break;
    case INT4: {
        float r = nearest ? rintf(m) : floorf(m);
        i = (int)fminf(r, (float)E.maxidx);
        break;
    }
    default: {  // E3M0: zero, then 2^-2 .. 2^4, no subnormals
        if (m < 0.25f) {
            i = nearest ? (m > 0.125f ? 1 : 0) : 0;
        } else {
            uint32_t u = fbits(m);
            if (nearest) u += 0x3fffffu + ((u >> 23) & 1u);
            i = (int)(u >> 23) - 124;
        }
        break;
    }
    }
    return i < E.maxidx ? i : E.maxidx;
}

__device__ __forceinline__ float grid_value(const Elem& E, int idx) {
    switch (E.kind) {
    case E2M1: return mf_value<1, 1>(idx);
    case E2M3: return mf_value<3, 1>(idx);
    case E3M2: return mf_value<2, 3>(idx);
    case E4M3: return mf_value<3, 7>(idx);
    case E5M2: return mf_value<2, 15>(idx);
    case INT4: return (float)idx;
    default: return idx == 0 ? 0.f : bitsf((uint32_t)(idx + 124) << 23);
    }
}

// E2M1 code of v (already divided by its scale) under stochastic rounding,
// from its bits.  Between neighbours lo <= |v| < hi the step is 2^(E-1) for
// |v| = 2^E (1 + m 2^-23) in [1, 6) and 0.5 below 1, so (|v| - lo) / step * 2^16
// is the bits below the code's mantissa bit over 64 ([1, 6)), the mantissa
// over 128 ([0.5, 1)) or |v| 2^17 (below 0.5): go up iff r16 is below it.
// |v| >= 6 (and Inf, NaN) takes the largest code.
__device__ __forceinline__ int sr_e2m1(float v, uint32_t r16) {
    const uint32_t b = fbits(v), u = b & 0x7fffffffu;
    int idx;
    if (u >= 0x40c00000u) idx = 7;
    else if (u >= 0x3f800000u) idx = (int)((u >> 22) - 252u) + ((r16 << 6) < (u & 0x3fffffu) ? 1 : 0);
    else if (u >= 0x3f000000u) idx = 1 + ((r16 << 7) < (u & 0x7fffffu) ? 1 : 0);
    else idx = (float)r16 < bitsf(u) * 131072.0f ? 1 : 0;
    return (int)((b >> 31) << 3) | idx;
}

// round v (already divided by its scale) to a code.  SR_BITS: E2M1 stochastic
// rounding by sr_e2m1 (same codes as the grid search below; a kernel that
// unrolls many elements and rarely takes that path keeps its code smaller
// without it)
template <bool SR_BITS = true>
__device__ __forceinline__ int encode(const Elem& E, int mode, float v, uint32_t r16) {
    if constexpr (SR_BITS)
        if (E.kind == E2M1 && mode == SR) return sr_e2m1(v, r16);
    bool neg = (fbits(v) >> 31) != 0;
    float m = fabsf(v);
    if (E.kind == INT4 && E.asym && neg) m = 0.f;
    int idx;
    if (!(m < E.qmax)) {
        idx = E.maxidx;
    } else if (mode == RTNE) {
        idx = grid_index(E, m, true);
    } else {
        int lo = grid_index(E, m, false);
        float a = grid_value(E, lo);
        if (mode == SR) {
            float step = grid_value(E, lo + 1) - a;           // a power of two
            float f = (m - a) * (1.0f / step);                // exact
            idx = ((float)r16 < f * 65536.0f) ? lo + 1 : lo;
        } else {
            idx = (neg && !(E.kind == INT4 && E.asym)) ? lo : (m > a ? lo + 1 : lo);
        }
    }
    if (E.kind == INT4) return E.asym ? idx : ((neg ? -idx : idx) & 0xf);
    return ((int)neg << (E.bits - 1)) | idx;
}

// bytes of one row of codes: 4-bit codes two per byte, 6-bit codes as a
// bit stream (4 per 3 bytes), 8-bit codes one per byte
__host__ __device__ inline int64_t code_row_bytes(int bits, int64_t cols) {
    return bits == 8 ? cols : bits == 6 ? cols * 3 / 4 : cols / 2;
}

__device__ __forceinline__ float decode(const Elem& E, int code) {
    if (E.kind == INT4) {
        if (E.asym) return (float)(code & 0xf);
        return (float)((code & 8) ? (code & 0xf) - 16 : (code & 0xf));
    }
    int sb = E.bits - 1;
    float mag = grid_value(E, code & ((1 << sb) - 1));
    return ((code >> sb) & 1) ? -mag : mag;
}

__device__ __forceinline__ bool finitef(float f);

// ---- scales -----------------------------------------------------------------
// E8M0 exponent of a block with largest magnitude amax, clamped to [-127, 127]
__device__ __forceinline__ int e8m0_exp(int rule, float tau, const Elem& E, float amax) {
    if (!(amax > 0.f)) return -127;
    if (!finitef(amax)) return 127;   // a block maximum that overflowed (e.g. an offset of +-FLT_MAX)
    int e;
    if (rule == RULE_FLOOR) e = flog2(amax) - E.emax;
    else e = e_ceil(amax, rule == RULE_CEIL ? E.qmax : tau);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// unsigned fp8 scale with 3 mantissa bits: UE4M3 (bias 7, max code 0x7E) or
// UE5M3 (bias 15, max code 0xFE); nearest-even, saturating; t >= 0
__device__ __forceinline__ int fp8_code(bool ue5, float t) {
    int c = ue5 ? mf_index<3, 15>(t, true) : mf_index<3, 7>(t, true);
    int mx = ue5 ? 0xfe : 0x7e;
    if (!(t < 1e30f)) return mx;
    return c < mx ? c : mx;
}

__device__ __forceinline__ float fp8_value(bool ue5, int code) {
    return ue5 ? mf_value<3, 15>(code) : mf_value<3, 7>(code);
}

// ---- bf16 -----------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return bitsf(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return bitsf(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return bitsf((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = fbits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// largest bf16 <= f
__device__ __forceinline__ uint16_t bf16_floor(float f) {
    uint32_t u = fbits(f);
    uint16_t h = (uint16_t)(u >> 16);
    if ((u & 0xffffu) && (u >> 31)) h = (uint16_t)(h + 1);
    return h;
}

__device__ __forceinline__ bool finitef(float f) { return (fbits(f) & 0x7f800000u) != 0x7f800000u; }

// ---- Philox4x32-10 ------------------------------------------------------------
// counter-based generator of Salmon et al. (SC'11): 10 rounds of two 32x32
// multiplies, Weyl key schedule
__device__ __forceinline__ void philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                         uint32_t k0, uint32_t k1, uint32_t out[4]) {
#pragma unroll
    for (int i = 0; i < 10; i++) {
        // each 32 x 32 -> 64-bit product as one 64-bit multiply of
        // zero-extended operands (one v_mad_u64_u32 instead of a low and a
        // high multiply)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// 8 consecutive 16-bit draws for logical indices 8j .. 8j+7
__device__ __forceinline__ void draws8(uint64_t seed, uint64_t off, uint64_t j, uint32_t r[8]) {
    uint32_t w[4];
    philox10((uint32_t)j, (uint32_t)(j >> 32), (uint32_t)off, (uint32_t)(off >> 32),
             (uint32_t)seed, (uint32_t)(seed >> 32), w);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        r[2 * i] = w[i] & 0xffffu;
        r[2 * i + 1] = w[i] >> 16;
    }
}

__device__ __forceinline__ uint32_t draw1(uint64_t seed, uint64_t off, uint64_t idx) {
    uint32_t w[4];
    uint64_t j = idx >> 3;
    philox10((uint32_t)j, (uint32_t)(j >> 32), (uint32_t)off, (uint32_t)(off >> 32),
             (uint32_t)seed, (uint32_t)(seed >> 32), w);
    uint32_t x = w[(idx >> 1) & 3];
    return (idx & 1) ? (x >> 16) : (x & 0xffffu);
}

// ---- wavefront reductions over aligned groups of G lanes (G | 64) ------------
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
template <int G>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}
template <int G>
__device__ __forceinline__ int group_and(int v) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v &= __shfl_xor(v, o, 64);
    return v;
}

// runtime group size (power of two <= 64)
__device__ __forceinline__ float group_max_rt(float v, int g) {
    for (int o = 1; o < g; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float group_min_rt(float v, int g) {
    for (int o = 1; o < g; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int group_and_rt(int v, int g) {
    for (int o = 1; o < g; o <<= 1) v &= __shfl_xor(v, o, 64);
    return v;
}

// ---- statistics partials -------------------------------------------------------
struct StatPart {
    double sig2, err2;
    unsigned long long nonzero, flushed, zero_blocks, pad;
};
static_assert(sizeof(StatPart) == 48, "a statistics partial is three 16-byte words");

// another lane's value under a DPP control that gives every lane a source
// (quad permutations, row mirrors): a VALU move, no LDS round trip
template <int CTRL>
__device__ __forceinline__ uint32_t lane_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ unsigned long long lane_mov(unsigned long long v) {
    return ((unsigned long long)lane_mov<CTRL>((uint32_t)(v >> 32)) << 32) | lane_mov<CTRL>((uint32_t)v);
}
template <int CTRL>
__device__ __forceinline__ double lane_mov(double v) {
    return __longlong_as_double((long long)lane_mov<CTRL>((unsigned long long)__double_as_longlong(v)));
}

// V_PERMLANE16_SWAP / V_PERMLANE32_SWAP on two copies a, b of a value:
// afterwards a holds the lower and b the upper partner's value (rows R lanes
// apart) in every lane
template <int R>
__device__ __forceinline__ void swap_rows(uint32_t& a, uint32_t& b) {
    if constexpr (R == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    }
}
// lower + upper partner (R lanes apart), the same bits in both lanes
template <int R, typename T>
__device__ __forceinline__ T row_pair_sum(T v) {
    if constexpr (sizeof(T) == 4) {
        uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
        swap_rows<R>(a, b);
        return __builtin_bit_cast(T, a) + __builtin_bit_cast(T, b);
    } else {
        const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
        uint32_t al = (uint32_t)u, bl = al, ah = (uint32_t)(u >> 32), bh = ah;
        swap_rows<R>(al, bl);
        swap_rows<R>(ah, bh);
        return __builtin_bit_cast(T, ((unsigned long long)ah << 32) | al) +
               __builtin_bit_cast(T, ((unsigned long long)bh << 32) | bl);
    }
}

// Sum over the 64 lanes, the same bits in every lane: pairs (quad_perm
// [1,0,3,2]), quads ([2,3,0,1]), the two quads of each 8 (half-row mirror),
// the two halves of each row of 16 (row mirror), then rows 16 and 32 apart
// (row swaps).  Every step adds two partners' values, which both get the
// same sum (addition is commutative), so the tree and the result are fixed.
// All 64 lanes must be active.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    v += lane_mov<0xB1>(v);
    v += lane_mov<0x4E>(v);
    v += lane_mov<0x141>(v);
    v += lane_mov<0x140>(v);
    v = row_pair_sum<16>(v);
    v = row_pair_sum<32>(v);
    return v;
}

// Workgroup sums of the per-thread statistics, valid in thread 0.  Wave sums,
// then the waves in index order: the result does not depend on timing.  C is
// the type the per-thread counts are summed in within a wave (32 bits where a
// workgroup's counts are known to fit).
template <int NT, typename C = unsigned long long>
__device__ __forceinline__ StatPart block_sum(double s2, double e2, C nz, C fl, C zb) {
    __shared__ double sh_d[2][NT / 64];
    __shared__ unsigned long long sh_u[3][NT / 64];
    s2 = wave_sum(s2);
    e2 = wave_sum(e2);
    nz = wave_sum(nz);
    fl = wave_sum(fl);
    zb = wave_sum(zb);
    int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) {
        sh_d[0][w] = s2; sh_d[1][w] = e2;
        sh_u[0][w] = nz; sh_u[1][w] = fl; sh_u[2][w] = zb;
    }
    __syncthreads();
    StatPart p;
    p.sig2 = 0; p.err2 = 0; p.nonzero = 0; p.flushed = 0; p.zero_blocks = 0; p.pad = 0;
    if (threadIdx.x == 0) {
        for (int i = 0; i < NT / 64; i++) {
            p.sig2 += sh_d[0][i]; p.err2 += sh_d[1][i];
            p.nonzero += sh_u[0][i]; p.flushed += sh_u[1][i]; p.zero_blocks += sh_u[2][i];
        }
    }
    return p;
}

template <int NT, typename C = unsigned long long>
__device__ __forceinline__ void block_stats(double s2, double e2, C nz, C fl, C zb, StatPart* dst) {
    const StatPart p = block_sum<NT, C>(s2, e2, nz, fl, zb);
    if (threadIdx.x == 0) *dst = p;
}

}  // namespace mxd
