// mx_kernels.hpp -- launch interface between the C ABI (api.hip) and the
// kernel translation units.  Internal to libmx.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.hpp"

namespace mxk {

// Everything a quantization launch needs.  Device pointers except where noted.
struct QParams {
    const void* x;
    int64_t rows, cols, ld;        // ld in elements
    int in_bf16;
    uint8_t* codes;
    uint8_t* scales;
    uint16_t* offsets;
    uint8_t* macro;
    const float* tensor_scale;     // NVFP4 g, produced by the pre-pass
    const int32_t* ref_exp;        // E3M0 e_ref, produced by the pre-pass
    void* dq;                      // nullable
    int dq_bf16;
    mxd::StatPart* parts;          // nullable: one partial per workgroup
    float* amax_parts;             // pre-pass mode: one max per workgroup
    int elem, asym, scale, rule, round;
    int br, bc, had, macro_cols;
    float tau;
    uint64_t seed, off;
};

constexpr int NT = 256;   // threads per workgroup for the streaming kernels

// row blocks (block_rows == 1): generic kernel; returns number of workgroups
int64_t rows_grid(const QParams& p);
hipError_t launch_rows(const QParams& p, bool amax_only, hipStream_t s);
// the E2M1 / E8M0 / RTNE row path on the hardware FP4 converter
bool rows_fast_ok(const QParams& p);
int64_t rows_fast_grid(const QParams& p);   // upper bound of the grid launch_rows_fast uses
hipError_t launch_rows_fast(const QParams& p, hipStream_t s, int64_t* grid);
// Several tensors of one such format and input dtype in one launch.  The
// caller fills x, codes, scales, parts (when p.parts is set: room for nb
// partials) and nchunks (16-byte chunks of input, nonzero) of job[0, count);
// the launcher sets b0 and nb, the workgroups each job takes.  *grid: the
// workgroups launched.
constexpr int MANY_MAX = 8;
struct FastJob {
    const void* x;
    uint8_t* codes;
    uint8_t* scales;
    mxd::StatPart* parts;
    int64_t nchunks, b0, nb;
};
struct FastMany {
    FastJob job[MANY_MAX];
    int count;
};
hipError_t launch_rows_fast_many(const QParams& p, FastMany& m, hipStream_t s, int64_t* grid);
// MXFP8 rows (E4M3 / E5M2 elements, E8M0 scales on 1 x 32 blocks, to nearest,
// dense) on the hardware FP8 converter
bool rows_fp8_ok(const QParams& p);
int64_t rows_fp8_grid(const QParams& p);    // upper bound of the grid launch_rows_fp8 uses
hipError_t launch_rows_fp8(const QParams& p, hipStream_t s, int64_t* grid);
// MXFP6 rows (E2M3 / E3M2, E8M0 scales on 1 x 32 blocks, to nearest, dense)
// on the hardware FP6 pack converter
bool rows_fp6_ok(const QParams& p);
int64_t rows_fp6_grid(const QParams& p);    // upper bound of the grid launch_rows_fp6 uses
hipError_t launch_rows_fp6(const QParams& p, hipStream_t s, int64_t* grid);
// the other E2M1 round-to-nearest row formats on the hardware FP4 converter
// (fp8 block scales, block Hadamard rotation, macro-block scales)
bool rows_hw_ok(const QParams& p);
int64_t rows_hw_grid(const QParams& p);     // upper bound of the grid launch_rows_hw uses
hipError_t launch_rows_hw(const QParams& p, hipStream_t s, int64_t* grid);
// column (b x 1) and 2D (b x b) blocks
int64_t tiles_grid(const QParams& p);
hipError_t launch_tiles(const QParams& p, hipStream_t s);
// tensor abs-max pre-pass (after the rotation, if any): amax_grid bounds the
// number of per-workgroup maxima; launch_amax reports the number written
int64_t amax_grid(const QParams& p);
hipError_t launch_amax(const QParams& p, hipStream_t s, int64_t* grid);
// finalize: tensor scale / reference exponent from the per-workgroup maxima
hipError_t launch_tensor_scale(const float* parts, int64_t n, int scale_kind, float qmax,
                               float* tensor_scale, int32_t* ref_exp, hipStream_t s);
// finalize: statistics from per-workgroup partials, fixed order
hipError_t launch_stats_final(const mxd::StatPart* parts, int64_t n, int64_t nelem, void* out,
                              hipStream_t s);
// the same for up to MANY_MAX partial sets in one launch, one workgroup each
struct FinalJob {
    const mxd::StatPart* parts;
    int64_t n, nelem;
    void* out;
};
struct FinalMany {
    FinalJob job[MANY_MAX];
};
hipError_t launch_stats_final_many(const FinalMany& m, int count, hipStream_t s);
// dequantize
hipError_t launch_dequant(const QParams& p, hipStream_t s);
// QSNR partials between two tensors
int64_t qsnr_grid(int64_t n);
hipError_t launch_qsnr(int bf16, const void* a, const void* b, int64_t n, mxd::StatPart* parts,
                       hipStream_t s);
// block-scaled GEMM; element codes E2M1, E2M3 or E3M2 for either operand
bool gemm_elem_ok(int elem);
hipError_t launch_gemm(int ea, const uint8_t* a, const uint8_t* sa, int eb, const uint8_t* b, const uint8_t* sb,
                       void* c, int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s,
                       const uint8_t* ma = nullptr, const uint8_t* mb = nullptr);
// LDS-staged kernel for E8M0 1 x 32 operands of any element pair, K % 128 == 0
// (ma / mb: UE4M3 macro-block scales per 1 x 128, E2M1 operands only; nullable)
hipError_t launch_gemm_lds(int ea, const uint8_t* a, const uint8_t* sa, int eb, const uint8_t* b, const uint8_t* sb,
                           void* c, int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s,
                           const uint8_t* ma = nullptr, const uint8_t* mb = nullptr);
// E2M1 operands under E8M0 / UE4M3 / NVFP4 / UE5M3 scales on 1 x bc blocks
// (bc a multiple of 8), decoded to bf16; ta / tb: per-tensor scales or null;
// ma / mb: UE4M3 macro-block scales per 1 x 128 (E8M0 block scales on both
// operands, K % 128 == 0), nullable
bool gemm_upcvt_scale_ok(int scale);
hipError_t launch_gemm_upcvt(int sca, int bca, const uint8_t* a, const uint8_t* sa, const float* ta, int scb, int bcb,
                             const uint8_t* b, const uint8_t* sb, const float* tb, void* c, int64_t M, int64_t N,
                             int64_t K, int64_t ldc, int c_bf16, hipStream_t s, const uint8_t* ma = nullptr,
                             const uint8_t* mb = nullptr);

}  // namespace mxk
