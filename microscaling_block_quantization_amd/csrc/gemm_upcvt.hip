// gemm_upcvt.hip -- block-scaled FP4 GEMM for scales the matrix instruction
// does not take: C = deq(A) . deq(B)^T with E2M1 elements under UE4M3 (NVFP4,
// with its fp32 per-tensor scale, "Unveiling the Potential of Quantization
// with MXFP4", Sec. 2), UE5M3 ("Is Finer Better?", technical summary) or E8M0
// block scales over row blocks of 8 .. 256 elements.
//
// gfx950's scaled matrix instruction applies one power-of-two scale per 32
// K-values of a lane, so a 16-element block with a 4-bit-significand scale
// has no exact mapping onto it (an E2M1 value times such a scale needs up to
// six significant bits, beyond FP8, FP6 and FP4).  Here each lane decodes its
// codes to fp32, multiplies by the block scale and narrows to bf16 -- exactly,
// since the product has at most six significant bits -- and the bf16 products
// run on V_MFMA_F32_32X32X16_BF16.  (The scaled converts use only the exponent
// of their scale operand, so they apply E8M0 scales directly but not UE4M3 /
// UE5M3 ones: measured on gfx950.)
// The per-tensor scales multiply the fp32 result once at the end.
//
// Layout: a lane of the bf16 instruction supplies 8 K-values of its row.  The
// K order inside one instruction is free as long as A and B agree, so lane
// (row r, half h) takes K = k0 + 32 h + 8 j + (0..7) in the j-th of the four
// instructions of a 64-wide K step: the 16 code bytes of k0 + 32 h .. + 31,
// one load, and every group of 8 lies inside one block (blocks are multiples
// of 8 wide).
#include "mx_kernels.hpp"

namespace mxk {
using namespace mxd;

namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

// scale kinds of an operand
enum { UK_E8M0 = 0, UK_UE4M3 = 1, UK_UE5M3 = 2 };

struct UOperand {
    const uint8_t* codes;     // rows x K/2 bytes
    const uint8_t* scales;    // rows x K/bc bytes
    int kind, bc;
};

// value of a scale code: E8M0 2^(c - 127) (0xFF: NaN); UE4M3 / UE5M3 unsigned
// minifloats with 3 mantissa bits, bias 7 / 15 (0x7F / 0xFF: NaN)
__device__ __forceinline__ float uscale(uint32_t c, int kind) {
    if (kind == UK_E8M0) return c == 255u ? __uint_as_float(0x7fc00000u) : __uint_as_float(c ? c << 23 : 0x00400000u);
    if ((kind == UK_UE4M3 && c == 0x7fu) || c == 0xffu) return __uint_as_float(0x7fc00000u);
    const int bias = kind == UK_UE4M3 ? 7 : 15;
    const uint32_t e = c >> 3, m = c & 7u;
    if (e) return __uint_as_float(((e + 127u - (uint32_t)bias) << 23) | (m << 20));
    return (float)m * __uint_as_float((uint32_t)(127 + 1 - bias - 3) << 23);
}

// eight bf16 products of the codes in dword w times a power of two s: the
// scaled converts take only the exponent field of their scale operand
__device__ __forceinline__ bf8v decode8_pow2(uint32_t w, float s) {
    const bf2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    const bf2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    const bf2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    const bf2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    bf8v v;
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    return v;
}

// the same for any scale: the codes decoded to fp32, multiplied by s (exact:
// at most six significant bits) and narrowed to bf16 (exact for the same
// reason)
template <int BYTE>
__device__ __forceinline__ bf2v decode2(uint32_t w, float s) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BYTE);
    const f2v p = {q[0] * s, q[1] * s};
    return __builtin_convertvector(p, bf2v);
}
__device__ __forceinline__ bf8v decode8(uint32_t w, float s) {
    const bf2v p0 = decode2<0>(w, s), p1 = decode2<1>(w, s), p2 = decode2<2>(w, s), p3 = decode2<3>(w, s);
    bf8v v;
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    return v;
}

// the 4 operands (8 K-values each) of one row for the 64-wide K step at k0
__device__ __forceinline__ void load_row(bf8v (&o)[4], const UOperand& U, int64_t row, int64_t k0, int half,
                                         int64_t K) {
    const int64_t kb = k0 + 32 * half;                     // first K of this lane
    if (kb >= K) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 8; i++) o[j][i] = (__bf16)0.0f;
        return;
    }
    const uint4 w = *reinterpret_cast<const uint4*>(U.codes + row * (K / 2) + kb / 2);
    const uint8_t* srow = U.scales + row * (K / U.bc);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float sc = uscale(srow[(kb + 8 * j) / U.bc], U.kind);
        o[j] = U.kind == UK_E8M0 ? decode8_pow2(ww[j], sc) : decode8(ww[j], sc);
    }
}

// 4 waves of 64 x 64 outputs (2 x 2 tiles of 32 x 32), operands from global
// memory straight into registers
template <bool CBF16>
__global__ __launch_bounds__(256) void k_gemm_upcvt(UOperand A, UOperand B, const float* ta, const float* tb,
                                                    void* __restrict__ C, int64_t M, int64_t N, int64_t K,
                                                    int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, row = lane & 31;
    const int64_t m0 = (int64_t)blockIdx.y * 128 + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * 128 + (wave & 1) * 64;
    int64_t ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t a = m0 + 32 * i + row, b = n0 + 32 * i + row;
        ra[i] = a < M ? a : M - 1;
        rb[i] = b < N ? b : N - 1;
    }
    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    for (int64_t k0 = 0; k0 < K; k0 += 64) {
        bf8v av[2][4], bv[2][4];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            load_row(av[i], A, ra[i], k0, half, K);
            load_row(bv[i], B, rb[i], k0, half, K);
        }
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i][q], bv[j][q], acc[i][j], 0, 0, 0);
    }

    const float g = (ta ? *ta : 1.0f) * (tb ? *tb : 1.0f);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t n = n0 + 32 * j + row;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + 32 * i + 8 * (r / 4) + 4 * half + (r % 4);
                if (m >= M) continue;
                const float v = acc[i][j][r] * g;
                if constexpr (CBF16) static_cast<uint16_t*>(C)[m * ldc + n] = bf16_rne(v);
                else static_cast<float*>(C)[m * ldc + n] = v;
            }
        }
}

int ukind(int scale) { return scale == SC_E8M0 ? UK_E8M0 : scale == SC_UE5M3 ? UK_UE5M3 : UK_UE4M3; }

}  // namespace

bool gemm_upcvt_scale_ok(int scale) {
    return scale == SC_E8M0 || scale == SC_UE4M3 || scale == SC_NVFP4 || scale == SC_UE5M3;
}

hipError_t launch_gemm_upcvt(int sca, int bca, const uint8_t* a, const uint8_t* sa, const float* ta, int scb, int bcb,
                             const uint8_t* b, const uint8_t* sb, const float* tb, void* c, int64_t M, int64_t N,
                             int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (!gemm_upcvt_scale_ok(sca) || !gemm_upcvt_scale_ok(scb) || bca % 8 || bcb % 8 || K % 32)
        return hipErrorInvalidValue;
    const UOperand A = {a, sa, ukind(sca), bca};
    const UOperand B = {b, sb, ukind(scb), bcb};
    dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
    if (c_bf16) k_gemm_upcvt<true><<<grid, 256, 0, s>>>(A, B, ta, tb, c, M, N, K, ldc);
    else k_gemm_upcvt<false><<<grid, 256, 0, s>>>(A, B, ta, tb, c, M, N, K, ldc);
    return hipGetLastError();
}

}  // namespace mxk
