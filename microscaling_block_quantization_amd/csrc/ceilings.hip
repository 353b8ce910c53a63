// ceilings.hip -- context kernels for the measurement (libmx_ceilings.so,
// include/mx_ceilings.h): a device copy, a read-mostly stream with the
// quantizer's byte mix, a loop of the block-scaled FP4 matrix instruction
// fed from LDS like the tiled GEMM, and the GEMM's LDS-DMA operand stream on
// its own.  Nothing here is part of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mx_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(NT) void k_read4_write1(const u32x4* __restrict__ src, uint32_t* __restrict__ dst,
                                                     int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const u32x4 w = __builtin_nontemporal_load(src + i);
        __builtin_nontemporal_store(w.x ^ w.y ^ w.z ^ w.w, dst + i);
    }
}

int64_t stream_grid(int64_t n) {
    const int64_t g = (n + NT - 1) / NT;
    return g < 8192 ? g : 8192;
}

// The matrix-instruction loop.  LDS holds 32 KiB of operand bytes: the first
// 16 KiB serve A fragments, the rest B fragments.  Per substep a wave reads
// 4 A and 2 B fragments (ds_read_b128; lane l at row l%32 of a 32-row block
// whose rows are 64 bytes apart, 16-byte chunk 2*t + l/32, XOR-swizzled by row
// so that the reads are free of bank conflicts) and issues 8 instructions.
// The fragment blocks advance with the iteration so that operands change
// every substep, as in a GEMM.
constexpr int LOOP_WAVES = 8;
constexpr int LOOP_LDS = 32768;

__device__ __forceinline__ v8i op8(u32x4 w) {
    v8i v;
    v[0] = (int)w.x; v[1] = (int)w.y; v[2] = (int)w.z; v[3] = (int)w.w;
    v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
    return v;
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (((row >> 1) & 3) ^ ((row >> 3) & 1)); }

// one 64-wide K substep T of iteration `it`: 6 operand reads, 8 instructions
template <int T>
__device__ __forceinline__ void loop_substep(const uint8_t* lds, v16f (&acc)[4][2], int64_t it, int wave, int row,
                                             int half) {
    const int sc = 0x7f7f7f7f;    // E8M0 127 = 2^0 in every byte
    u32x4 a[4], b[2];
    const int base = (int)((it * 2 + T + wave) & 7);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int blk = (base + i) & 7, r = blk * 32 + row;
        a[i] = *reinterpret_cast<const u32x4*>(lds + r * 64 + (swz(r, 2 * T + half) << 4));
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int blk = (base + 4 + j) & 7, r = blk * 32 + row;
        b[j] = *reinterpret_cast<const u32x4*>(lds + 16384 + r * 64 + (swz(r, 2 * T + half) << 4));
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8(a[i]), op8(b[j]), acc[i][j], 4, 4, 2 * T,
                                                                       sc, 2 * T, sc);
}

__global__ __launch_bounds__(64 * LOOP_WAVES, 1) void k_mfma_loop(const u32x4* __restrict__ ops, float* out,
                                                                 int64_t iters) {
    // 96 KiB reserved so that one workgroup occupies a CU (only 32 KiB is used)
    __shared__ __attribute__((aligned(16))) uint8_t lds[3 * LOOP_LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < LOOP_LDS / 16; i += 64 * LOOP_WAVES) reinterpret_cast<u32x4*>(lds)[i] = ops[i];
    __syncthreads();
    const int row = lane & 31, half = lane >> 5;
    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    // 8 row blocks of 32 rows x 64 bytes per operand half
    for (int64_t it = 0; it < iters; it++) {
        loop_substep<0>(lds, acc, it, wave, row, half);
        loop_substep<1>(lds, acc, it, wave, row, half);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) s += acc[i][j][r];
    out[(int64_t)blockIdx.x * 64 * LOOP_WAVES + tid] = s;
}

// The LDS-DMA stream of the tiled GEMM without its arithmetic: each
// workgroup of 8 waves moves `stages` stages of 32 KiB from global memory
// into a 4-slot LDS ring with buffer_load_dwordx4 ... lds (16 bytes per lane).
// A stage is 512 rows x 64 bytes of a window of 512 rows x 2048 bytes (the
// 256 + 256 operand rows of one 256 x 256 output tile at K = 4096 in FP4):
// each instruction moves 16 rows x 64 bytes, 4 per wave per stage; two stages
// stay in flight and a barrier closes each stage, as in the GEMM.  The windows
// (1 MiB each) are shared round robin by the workgroups, so after the first
// pass they are read from the L2 / Infinity Cache, as the GEMM's panels are.
constexpr int DMA_WAVES = 8;
constexpr int DMA_STAGE = 32768;
typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(64 * DMA_WAVES, 1) void k_lds_dma(const uint8_t* __restrict__ src, int nwin, int stages,
                                                              uint32_t* out) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[4 * DMA_STAGE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* win = src + (size_t)(blockIdx.x % nwin) * (1u << 20);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(win), (short)0, 1 << 20,
                                                                       0x00020000);
    uint32_t acc = 0;
    for (int st = 0; st < stages; st++) {
        uint8_t* slot = ring + (st & 3) * DMA_STAGE;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int g = wave * 4 + k;                   // 16-row piece 0 .. 31
            const int vo = (g * 16 + lane / 4) * 2048 + (st & 31) * 64 + (lane & 3) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slot + g * 1024), 16, vo, 0, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // this wave's stage st - 2 has landed
        __syncthreads();
        acc += ring[(threadIdx.x * 64 + st * 4) % (4 * DMA_STAGE)];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    acc += ring[(threadIdx.x * 64) % (4 * DMA_STAGE)];
    out[(int64_t)blockIdx.x * 64 * DMA_WAVES + threadIdx.x] = acc;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

int mxc_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || !aligned16(src) || !aligned16(dst)) return 1;
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return 0;
    k_copy<<<(unsigned)stream_grid(n), NT, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int mxc_read4_write1(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || !aligned16(src) || !aligned16(dst)) return 1;
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return 0;
    k_read4_write1<<<(unsigned)stream_grid(n), NT, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), static_cast<uint32_t*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int mxc_mfma_loop_grid(void) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    return cus;
}

double mxc_mfma_loop_flops(int grid, int64_t iters) {
    return 2.0 * 32 * 32 * 64 * 16.0 * LOOP_WAVES * (double)grid * (double)iters;
}

int mxc_mfma_loop(const void* operands, float* out, int grid, int64_t iters, void* stream) {
    if (!operands || !out || grid <= 0 || iters <= 0 || !aligned16(operands)) return 1;
    k_mfma_loop<<<(unsigned)grid, 64 * LOOP_WAVES, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(operands), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int mxc_lds_dma(const void* src, size_t src_bytes, uint32_t* out, int grid, int stages, void* stream) {
    if (!src || !out || grid <= 0 || stages <= 0 || src_bytes < (1u << 20) || src_bytes % (1u << 20) ||
        !aligned16(src))
        return 1;
    const int nwin = (int)(src_bytes >> 20);
    k_lds_dma<<<(unsigned)grid, 64 * DMA_WAVES, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint8_t*>(src), nwin, stages, out);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
