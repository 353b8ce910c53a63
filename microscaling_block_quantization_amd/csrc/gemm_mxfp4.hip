// gemm_mxfp4.hip -- block-scaled FP4 GEMM C = deq(A) . deq(B)^T on gfx950.
//
// The pages describe the consumer of MXFP4 data as a dot-product unit that
// resolves each block's effective scale, aligns block partial sums and adds
// them ("Unveiling the Potential of Quantization with MXFP4", Sec. 3, Fig. 4;
// the A.B^T product with block scales, Sec. 4, Fig. 5).  On CDNA4 that unit is
// the V_MFMA_SCALE_F32_32X32X64_F8F6F4 instruction with E2M1 operands: every
// lane supplies 32 consecutive K values of one row (16 bytes, even element in
// the low nibble) plus the E8M0 scale of exactly that 32-element block, so an
// MXFP4 block maps onto one lane's operand without any repacking.  Output
// layout of the 32x32 fp32 accumulator: lane l, register r holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "mx_kernels.hpp"

namespace mxk {
using namespace mxd;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int TM = 128, TN = 128, TK = 128;

__device__ __forceinline__ v8i as_operand(uint4 w) {
    v8i v;
    v[0] = (int)w.x; v[1] = (int)w.y; v[2] = (int)w.z; v[3] = (int)w.w;
    v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
    return v;
}

template <bool CBF16>
__global__ __launch_bounds__(256) void k_gemm_simple(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                     void* __restrict__ C, int64_t M, int64_t N, int64_t K, int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, row = lane & 31;
    const int64_t m0 = (int64_t)blockIdx.y * TM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * TN + (wave & 1) * 64;
    const int64_t rowb = K / 2, kblocks = K / 32;

    int64_t ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        int64_t a = m0 + 32 * i + row, b = n0 + 32 * i + row;
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

    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        uint4 av[2][2], bv[2][2];
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                av[i][kk] = *reinterpret_cast<const uint4*>(A + ra[i] * rowb + (k0 + 64 * kk + 32 * half) / 2);
                bv[i][kk] = *reinterpret_cast<const uint4*>(B + rb[i] * rowb + (k0 + 64 * kk + 32 * half) / 2);
            }
            // the four E8M0 scales of this row over the 128-wide K step; this
            // lane's block of chunk kk sits in byte 2*kk after the shift
            sa[i] = (int)(*reinterpret_cast<const uint32_t*>(SA + ra[i] * kblocks + k0 / 32) >> (8 * half));
            sb[i] = (int)(*reinterpret_cast<const uint32_t*>(SB + rb[i] * kblocks + k0 / 32) >> (8 * half));
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    as_operand(av[i][0]), as_operand(bv[j][0]), acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    as_operand(av[i][1]), as_operand(bv[j][1]), acc[i][j], 4, 4, 2, sa[i], 2, sb[j]);
            }
    }

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
                if constexpr (CBF16) static_cast<uint16_t*>(C)[m * ldc + n] = bf16_rne(acc[i][j][r]);
                else static_cast<float*>(C)[m * ldc + n] = acc[i][j][r];
            }
        }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c,
                       int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    if (c_bf16) k_gemm_simple<true><<<grid, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
    else k_gemm_simple<false><<<grid, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
    return hipGetLastError();
}

}  // namespace mxk
