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

bool rows_fast_ok(const QParams&) { return false; }
int64_t rows_fast_grid(const QParams& p) { return rows_grid(p); }
hipError_t launch_rows_fast(const QParams& p, hipStream_t s) { return launch_rows(p, false, s); }

hipError_t launch_amax(const QParams& p, hipStream_t s) { return launch_rows(p, true, s); }

}  // namespace mxk
