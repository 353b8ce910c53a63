// misc.hip -- tensor-scale pre-pass finalize, deterministic statistics
// finalize, dequantize and the QSNR reduction for gfx950.
//
// QSNR follows eq. (1) / (2) of "Unveiling the Potential of Quantization with
// MXFP4" (Sec. 3): ten times log10 of ||A||_F^2 over ||A - A_q||_F^2.  The two
// squared norms accumulate in float64; per-workgroup partials are combined in
// a fixed order so repeated runs give identical bits.
#include "mx_kernels.hpp"

namespace mxk {
using namespace mxd;

namespace {

// one workgroup: max over the per-workgroup maxima, then the NVFP4 per-tensor
// scale g = amax / (Qmax * 448) ("Unveiling ... MXFP4", Sec. 2: NVFP4's third
// component) or the E3M0 reference exponent (smallest e with Qmax 2^e >= amax)
__global__ __launch_bounds__(NT) void k_tensor_scale(const float* parts, int64_t n, int kind, float qmax,
                                                     float* ts, int32_t* re) {
    __shared__ float sh[NT / 64];
    float a = 0.f;
    // eight independent loads in flight per thread
    constexpr int U = 8;
    for (int64_t base = threadIdx.x; base < n; base += (int64_t)NT * U) {
        float q[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t i = base + (int64_t)u * NT;
            q[u] = i < n ? parts[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; u++) a = fmaxf(a, q[u]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = sh[0];
        for (int i = 1; i < NT / 64; i++) m = fmaxf(m, sh[i]);
        if (kind == SC_NVFP4) *ts = m > 0.f ? m / (qmax * 448.0f) : 1.0f;
        if (kind == SC_E3M0) *re = m > 0.f ? e_ceil(m, qmax) : 0;
    }
}

struct StatsOut {
    double sig2, err2;
    long long n, nonzero, flushed, zero_blocks;
};

// one workgroup adds n partials into *out
__device__ __forceinline__ void stats_final(const StatPart* parts, int64_t n, int64_t nelem, StatsOut* out) {
    double s2 = 0, e2 = 0;
    unsigned long long nz = 0, fl = 0, zb = 0;
    // each thread owns the partials t, t + NT, ...; eight of them are loaded
    // before any is added so the loads overlap
    constexpr int U = 8;
    for (int64_t base = threadIdx.x; base < n; base += (int64_t)NT * U) {
        StatPart q[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t i = base + (int64_t)u * NT;
            if (i < n) q[u] = parts[i];
            else q[u] = StatPart{0.0, 0.0, 0ull, 0ull, 0ull, 0ull};
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            s2 += q[u].sig2; e2 += q[u].err2; nz += q[u].nonzero; fl += q[u].flushed; zb += q[u].zero_blocks;
        }
    }
    // wave butterflies, then the waves in order: a fixed summation order
    const StatPart r = block_sum<NT>(s2, e2, nz, fl, zb);
    if (threadIdx.x == 0) {
        StatsOut o;
        o.sig2 = r.sig2; o.err2 = r.err2; o.n = nelem;
        o.nonzero = (long long)r.nonzero; o.flushed = (long long)r.flushed; o.zero_blocks = (long long)r.zero_blocks;
        *out = o;
    }
}

__global__ __launch_bounds__(NT) void k_stats_final(const StatPart* parts, int64_t n, int64_t nelem,
                                                    StatsOut* out) {
    stats_final(parts, n, nelem, out);
}

// workgroup i finalizes job i
__global__ __launch_bounds__(NT) void k_stats_final_many(FinalMany m) {
    const FinalJob& J = m.job[blockIdx.x];
    stats_final(J.parts, J.n, J.nelem, static_cast<StatsOut*>(J.out));
}

__device__ __forceinline__ int read_code(const uint8_t* row, int bits, int64_t c) {
    if (bits == 8) return row[c];
    if (bits == 4) return (row[c >> 1] >> ((c & 1) * 4)) & 0xf;
    const int64_t bit = 6 * c;
    // the second byte is read only when the code crosses into it, so the last
    // code of the last row never reads past the buffer
    uint32_t lo = row[bit >> 3], hi = (bit & 7) > 2 ? row[(bit >> 3) + 1] : 0u;
    return (int)(((lo | (hi << 8)) >> (bit & 7)) & 0x3f);
}

// 8 consecutive elements of one row per thread
__global__ __launch_bounds__(NT) void k_dequant(QParams p, void* y, int64_t ld, int out_bf16) {
    const Elem E = make_elem(p.elem, p.asym);
    const int64_t per_row = p.cols / 8;
    const int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (q >= p.rows * per_row) return;
    const int64_t r = q / per_row, c0 = (q - r * per_row) * 8;
    const int64_t crow = code_row_bytes(E.bits, p.cols);
    const uint8_t* row = p.codes + r * crow;
    const float g = p.scale == SC_NVFP4 ? *p.tensor_scale : 1.0f;
    const int eref = p.scale == SC_E3M0 ? *p.ref_exp : 0;
    const bool ue5 = p.scale == SC_UE5M3;
    const int64_t nbc = p.cols / p.bc;
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t c = c0 + i;
        const int64_t sidx = (r / p.br) * nbc + c / p.bc;
        const int sc = p.scales[sidx];
        const float val = decode(E, read_code(row, E.bits, c));
        float v;
        if (p.scale == SC_E8M0 || p.asym) {
            if (sc == 0xff) {
                v = __uint_as_float(0x7fc00000u);
            } else {
                v = val * pow2f(sc - 127);
                if (p.asym) v = v + bf16f(p.offsets[sidx]);
                if (p.macro_cols) v = v * fp8_value(false, p.macro[r * (p.cols / 128) + c / 128]);
            }
        } else if (p.scale == SC_E3M0) {
            v = sc == 0xff ? __uint_as_float(0x7fc00000u) : val * pow2f(eref - sc);
        } else {
            if (sc == (ue5 ? 0xff : 0x7f)) {
                v = __uint_as_float(0x7fc00000u);
            } else {
                v = val * fp8_value(ue5, sc);
                if (p.scale == SC_NVFP4) v = v * g;
            }
        }
        out[i] = v;
    }
    if (out_bf16) {
        uint16_t* dst = static_cast<uint16_t*>(y) + r * ld + c0;
        uint4 w;
        w.x = bf16_rne(out[0]) | ((uint32_t)bf16_rne(out[1]) << 16);
        w.y = bf16_rne(out[2]) | ((uint32_t)bf16_rne(out[3]) << 16);
        w.z = bf16_rne(out[4]) | ((uint32_t)bf16_rne(out[5]) << 16);
        w.w = bf16_rne(out[6]) | ((uint32_t)bf16_rne(out[7]) << 16);
        *reinterpret_cast<uint4*>(dst) = w;
    } else {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + r * ld + c0);
        dst[0] = make_float4(out[0], out[1], out[2], out[3]);
        dst[1] = make_float4(out[4], out[5], out[6], out[7]);
    }
}

constexpr int QSNR_ITEMS = 4096;   // elements per workgroup

__global__ __launch_bounds__(NT) void k_qsnr(int bf16, const void* a, const void* b, int64_t n,
                                             StatPart* parts) {
    double s2 = 0, e2 = 0;
    unsigned long long nz = 0, fl = 0;
    const int64_t base = (int64_t)blockIdx.x * QSNR_ITEMS;
    for (int i = threadIdx.x; i < QSNR_ITEMS; i += NT) {
        const int64_t k = base + i;
        if (k >= n) break;
        float x, y;
        if (bf16) {
            x = bf16f(static_cast<const uint16_t*>(a)[k]);
            y = bf16f(static_cast<const uint16_t*>(b)[k]);
        } else {
            x = static_cast<const float*>(a)[k];
            y = static_cast<const float*>(b)[k];
        }
        double xd = x, yd = y;
        s2 += xd * xd;
        e2 += (xd - yd) * (xd - yd);
        nz += (x != 0.f);
        fl += (x != 0.f && y == 0.f);
    }
    block_stats<NT>(s2, e2, nz, fl, 0ull, parts + blockIdx.x);
}

}  // namespace

hipError_t launch_tensor_scale(const float* parts, int64_t n, int kind, float qmax, float* ts,
                               int32_t* re, hipStream_t s) {
    k_tensor_scale<<<1, NT, 0, s>>>(parts, n, kind, qmax, ts, re);
    return hipGetLastError();
}

hipError_t launch_stats_final(const StatPart* parts, int64_t n, int64_t nelem, void* out, hipStream_t s) {
    k_stats_final<<<1, NT, 0, s>>>(parts, n, nelem, static_cast<StatsOut*>(out));
    return hipGetLastError();
}

hipError_t launch_stats_final_many(const FinalMany& m, int count, hipStream_t s) {
    if (count < 1 || count > MANY_MAX) return hipErrorInvalidValue;
    k_stats_final_many<<<count, NT, 0, s>>>(m);
    return hipGetLastError();
}

hipError_t launch_dequant(const QParams& p, hipStream_t s) {
    const int64_t n = p.rows * (p.cols / 8);
    if (n == 0) return hipSuccess;
    k_dequant<<<(n + NT - 1) / NT, NT, 0, s>>>(p, p.dq, p.ld, p.dq_bf16);
    return hipGetLastError();
}

int64_t qsnr_grid(int64_t n) { return (n + QSNR_ITEMS - 1) / QSNR_ITEMS; }

hipError_t launch_qsnr(int bf16, const void* a, const void* b, int64_t n, StatPart* parts, hipStream_t s) {
    const int64_t grid = qsnr_grid(n);
    if (grid == 0) return hipSuccess;
    k_qsnr<<<grid, NT, 0, s>>>(bf16, a, b, n, parts);
    return hipGetLastError();
}

}  // namespace mxk
