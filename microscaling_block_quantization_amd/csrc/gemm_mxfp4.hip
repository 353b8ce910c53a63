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

#ifndef GEMM_BK
#define GEMM_BK 128
#endif
#ifndef GEMM_D
#define GEMM_D 4
#endif

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

    // K advances 128 per step; a 32-element block past the end of K (K is a
    // multiple of 32 only) contributes zero codes under scale code 0
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        uint4 av[2][2], bv[2][2];
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            uint32_t ca[2], cb[2];
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const int64_t kb = k0 / 32 + 2 * kk + half;   // this lane's K block
                const bool in = kb < kblocks;
                av[i][kk] = in ? *reinterpret_cast<const uint4*>(A + ra[i] * rowb + kb * 16) : make_uint4(0, 0, 0, 0);
                bv[i][kk] = in ? *reinterpret_cast<const uint4*>(B + rb[i] * rowb + kb * 16) : make_uint4(0, 0, 0, 0);
                ca[kk] = in ? SA[ra[i] * kblocks + kb] : 0u;
                cb[kk] = in ? SB[rb[i] * kblocks + kb] : 0u;
            }
            // the scale of K block 2*kk + half in byte 2*kk: the op_sel value below
            sa[i] = (int)(ca[0] | (ca[1] << 16));
            sb[i] = (int)(cb[0] | (cb[1] << 16));
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


// ---------------------------------------------------------------------------
// Tiled kernel: 256 x 256 output tile per 256-thread workgroup (one wave per
// SIMD, each wave 128 x 128 = 4 x 4 MFMA tiles, 256 fp32 accumulators per
// lane).  K advances BK per stage; a stage holds the tile's A and B codes
// (256 rows x BK/2 bytes each) and their E8M0 scales (256 rows x BK/32
// bytes).  D stages form a ring in LDS: stage s + D - 1 is fetched by
// LDS-DMA (global_load_lds, 16 bytes per lane for codes, 4 for scales) while
// stage s is multiplied, so every load has D - 1 stages of MFMA work to land.
// The 16-byte chunks of a code row are XOR-swizzled so that the ds_read_b128
// operand reads of consecutive rows fall in distinct LDS bank groups.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int BM = 256, BN = 256;

template <int BK>
struct Geo {
    static constexpr int ROWB = BK / 2;            // code bytes per row per stage
    static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
    static constexpr int SPR = BK / 32;            // scale bytes per row per stage
    static constexpr int ST_A = BM * ROWB;
    static constexpr int ST_B = BN * ROWB;
    static constexpr int ST_S = 256 * SPR;
    static constexpr int STAGE = ST_A + ST_B + 2 * ST_S;
    // physical chunk of logical chunk c in row r
    static __device__ __forceinline__ int phys(int r, int c) {
        if constexpr (CPR == 8) return c ^ ((r & 7) ^ ((r >> 3) & 1));
        else return c ^ (((r >> 1) & 3) ^ ((r >> 3) & 1));
    }
};

__device__ __forceinline__ v8i op8(u32x4v w) {
    v8i v;
    v[0] = (int)w.x; v[1] = (int)w.y; v[2] = (int)w.z; v[3] = (int)w.w;
    v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
    return v;
}

// Buffer resources over one tile's operand panels: base = the tile's first
// row, size = its valid rows, so rows past M (or N) read as zero and every
// offset fits in 32 bits.  0x00020000: raw 32-bit data format.
struct Panels {
    __amdgpu_buffer_rsrc_t a, b, sa, sb;
    int rowb, kblocks;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel(const uint8_t* base, int64_t row0, int64_t nrows, int rowbytes) {
    const int64_t valid = nrows - row0 < 256 ? nrows - row0 : 256;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * rowbytes), (short)0, (int)(valid * rowbytes),
                                             0x00020000);
}

// LDS-DMA of one stage.  A wave-load writes 1 KiB of LDS, lane l at bytes
// [16 l, 16 l + 16), so each lane fetches the logical chunk that the swizzle
// stores at its position; the swizzle of row r depends on r mod 16 only.
template <int BK>
__device__ __forceinline__ void stage_dma(uint8_t* __restrict__ lds, const Panels& P, int s, int wave, int lane) {
    using G = Geo<BK>;
    constexpr int RPL = 1024 / G::ROWB;              // rows per wave-load
    constexpr int LOADS = G::ST_A / 1024 / 4;        // wave-loads per wave and operand
    const int rin = lane / G::CPR, pc = lane % G::CPR;
    const int vo0 = rin * P.rowb + (G::phys(rin, pc) << 4);            // even slots (RPL = 8) / all slots
    const int vo1 = rin * P.rowb + (G::phys(rin + 8, pc) << 4);        // odd slots when RPL = 8
#pragma unroll
    for (int j = 0; j < LOADS; j++) {
        const int slot = wave * LOADS + j;
        const int vo = (RPL == 8 && (slot & 1)) ? vo1 : vo0;
        const int so = slot * RPL * P.rowb + s * G::ROWB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(P.a, (lds_void*)(lds + slot * 1024), 16, vo, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(P.b, (lds_void*)(lds + G::ST_A + slot * 1024), 16, vo, so, 0, 0);
    }
    constexpr int DPR = G::SPR / 4;                   // scale dwords per row per stage
    constexpr int SLOADS = G::ST_S / 256 / 4;
    const int svo = (lane / DPR) * P.kblocks + (lane % DPR) * 4;
#pragma unroll
    for (int j = 0; j < SLOADS; j++) {
        const int slot = wave * SLOADS + j;
        const int so = (slot * 64 / DPR) * P.kblocks + s * G::SPR;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(P.sa, (lds_void*)(lds + G::ST_A + G::ST_B + slot * 256), 4, svo, so,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(P.sb, (lds_void*)(lds + G::ST_A + G::ST_B + G::ST_S + slot * 256), 4,
                                                 svo, so, 0, 0);
    }
}

// operands of one 64-wide K substep: four A and four B 16-byte fragments and
// the raw scale dwords of their rows
struct Ops {
    u32x4v a[4], b[4];
    uint32_t sa[4], sb[4];
};

template <int BK>
__device__ __forceinline__ void load_ops(Ops& o, const uint8_t* __restrict__ st, int t, int wm, int wn, int lrow,
                                         int half) {
    using G = Geo<BK>;
    // rows i*32 apart share the swizzle (it depends on r mod 16), so each
    // operand needs one lane address per substep and the four row tiles are
    // immediate offsets from it
    const int c = 2 * t + half;                      // this lane's 32-wide block in the stage
    const int ra = wm * 128 + lrow, rb = wn * 128 + lrow;
    const uint8_t* pa = st + ra * G::ROWB + (G::phys(ra, c) << 4);
    const uint8_t* pb = st + G::ST_A + rb * G::ROWB + (G::phys(rb, c) << 4);
    const uint8_t* qa = st + G::ST_A + G::ST_B + ra * G::SPR + 4 * (t >> 1);
    const uint8_t* qb = st + G::ST_A + G::ST_B + G::ST_S + rb * G::SPR + 4 * (t >> 1);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        o.a[i] = *reinterpret_cast<const u32x4v*>(pa + i * 32 * G::ROWB);
        o.b[i] = *reinterpret_cast<const u32x4v*>(pb + i * 32 * G::ROWB);
        o.sa[i] = *reinterpret_cast<const uint32_t*>(qa + i * 32 * G::SPR);
        o.sb[i] = *reinterpret_cast<const uint32_t*>(qb + i * 32 * G::SPR);
    }
}

// 16 MFMAs of one substep.  After the shift by 8*half this lane's scale byte
// (block 2t + half of the stage) is byte 2*(t&1): the op_sel value.
template <int T1>
__device__ __forceinline__ void mma(const Ops& o, v16f (&acc)[4][4], int half) {
    int xa[4], xb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        xa[i] = (int)(o.sa[i] >> (8 * half));
        xb[i] = (int)(o.sb[i] >> (8 * half));
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8(o.a[i]), op8(o.b[j]), acc[i][j], 4, 4,
                                                                       2 * T1, xa[i], 2 * T1, xb[j]);
}

// scheduling masks of __builtin_amdgcn_sched_group_barrier
constexpr int SG_VALU = 0x2, SG_MFMA = 0x8, SG_DSR = 0x100;

// One substep group in a fixed instruction order: MFMA k of `cur`, then LDS
// read k of the next operands, then DMA instruction k of a later stage, with
// a scheduling fence after each step.  Every DMA instruction holds the wave
// at the texture unit for a while and the MFMA in flight hides it; every LDS
// read has the rest of the group to land.
struct DmaSlot {
    uint8_t* lds;          // uniform LDS destination (goes to M0)
    const Panels* P;
    int s, wave, lane;
};

template <int BK>
__device__ __forceinline__ void dma_piece(const DmaSlot& d, int k) {
    using G = Geo<BK>;
    constexpr int RPL = 1024 / G::ROWB;
    constexpr int LOADS = G::ST_A / 1024 / 4;
    const int rin = d.lane / G::CPR, pc = d.lane % G::CPR;
    if (k < 2 * LOADS) {
        const int j = k >> 1, slot = d.wave * LOADS + j;
        const int vo = rin * d.P->rowb + (G::phys((RPL == 8 && (slot & 1)) ? rin + 8 : rin, pc) << 4);
        const int so = slot * RPL * d.P->rowb + d.s * G::ROWB;
        if (k & 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.P->b, (lds_void*)(d.lds + G::ST_A + slot * 1024), 16, vo, so, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.P->a, (lds_void*)(d.lds + slot * 1024), 16, vo, so, 0, 0);
    } else {
        constexpr int DPR = G::SPR / 4;
        constexpr int SLOADS = G::ST_S / 256 / 4;
        const int kk = k - 2 * LOADS, j = kk >> 1, slot = d.wave * SLOADS + j;
        const int svo = (d.lane / DPR) * d.P->kblocks + (d.lane % DPR) * 4;
        const int so = (slot * 64 / DPR) * d.P->kblocks + d.s * G::SPR;
        if (kk & 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.P->sb, (lds_void*)(d.lds + G::ST_A + G::ST_B + G::ST_S + slot * 256),
                                                     4, svo, so, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.P->sa, (lds_void*)(d.lds + G::ST_A + G::ST_B + slot * 256), 4,
                                                     svo, so, 0, 0);
    }
}

// LDS read k (0..11) of the operands of substep t: k = 0..3 A fragments,
// 4..7 B fragments, 8..11 scale dwords (A, B pairs)
template <int BK>
__device__ __forceinline__ void ops_piece(Ops& o, const uint8_t* __restrict__ st, int t, int wm, int wn, int lrow,
                                          int half, int k) {
    using G = Geo<BK>;
    const int c = 2 * t + half;
    const int ra = wm * 128 + lrow, rb = wn * 128 + lrow;
    if (k < 4) {
        o.a[k] = *reinterpret_cast<const u32x4v*>(st + ra * G::ROWB + (G::phys(ra, c) << 4) + k * 32 * G::ROWB);
    } else if (k < 8) {
        o.b[k - 4] = *reinterpret_cast<const u32x4v*>(st + G::ST_A + rb * G::ROWB + (G::phys(rb, c) << 4) +
                                                      (k - 4) * 32 * G::ROWB);
    } else {
        const int i = k - 8;
        o.sa[i] = *reinterpret_cast<const uint32_t*>(st + G::ST_A + G::ST_B + ra * G::SPR + 4 * (t >> 1) +
                                                      i * 32 * G::SPR);
        o.sb[i] = *reinterpret_cast<const uint32_t*>(st + G::ST_A + G::ST_B + G::ST_S + rb * G::SPR + 4 * (t >> 1) +
                                                      i * 32 * G::SPR);
    }
}

template <int BK, int T1, int NV>
__device__ __forceinline__ void substep(const Ops& cur, v16f (&acc)[4][4], Ops& nxt, const uint8_t* __restrict__ st,
                                      int t, int wm, int wn, int lrow, int half, const DmaSlot* d) {
    int xa[4], xb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        xa[i] = (int)(cur.sa[i] >> (8 * half));
        xb[i] = (int)(cur.sb[i] >> (8 * half));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; k++) {
        const int i = k >> 2, j = k & 3;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8(cur.a[i]), op8(cur.b[j]), acc[i][j], 4, 4,
                                                                   2 * T1, xa[i], 2 * T1, xb[j]);
        if (k < 12) ops_piece<BK>(nxt, st, t, wm, wn, lrow, half, k);
        if (k < NV) dma_piece<BK>(*d, k);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// wait until at most N vector-memory ops of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// all waves' DMA of a stage has landed (each wave waited for its own) and
// every wave has consumed its reads of the buffer about to be refilled, so a
// bare s_barrier suffices; a release fence would also wait for the DMA of the
// stages still in flight
__device__ __forceinline__ void bar() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// the stage handover: start the DMA of a later stage into `dma` while the
// last substep of the current stage multiplies and the first operands of the
// next stage are read from `nxt`.  The buffers are distinct restrict-qualified
// objects here, so the operand reads carry no dependence on the DMA.
template <int BK, int T1>
__device__ __forceinline__ void handover(const uint8_t* __restrict__ nxt, const Ops& cur, v16f (&acc)[4][4], Ops& o,
                                         int wm, int wn, int lrow, int half) {
    substep<BK, T1, 0>(cur, acc, o, nxt, 0, wm, wn, lrow, half, nullptr);
}

template <bool CBF16, int BK, int D>
__global__ __launch_bounds__(256, 1) void k_gemm_tiled(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                       const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                       void* __restrict__ C, int64_t M, int64_t N, int64_t K,
                                                       int64_t ldc) {
    using G = Geo<BK>;
    static_assert(D >= 3 && D <= 4, "ring depth: the handover waits for the next stage while D - 3 more are in flight");
    constexpr int NSUB = BK / 64;
    constexpr int L = 2 * (G::ST_A / 1024 / 4) + 2 * (G::ST_S / 256 / 4);   // DMA ops per wave per stage
    constexpr int CROW = 128 * 2 + 16;               // padded bf16 row of a wave's C tile in LDS
    static_assert(D * G::STAGE >= 4 * 128 * CROW, "C staging must fit in the ring");
    __shared__ __attribute__((aligned(16))) uint8_t smem[D * G::STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, lrow = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware, grouped tile order: workgroups are dealt to the 8 XCDs round
    // robin, so consecutive tiles of the grouped order go to one XCD and share
    // A and B panels in its L2
    const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
    const int T = tm * tn;
    int bid = blockIdx.x;
    if (T % 8 == 0) bid = (bid % 8) * (T / 8) + bid / 8;
    constexpr int GM = 8;
    const int group = bid / (GM * tn);
    const int first = group * GM;
    const int gsz = (tm - first) < GM ? (tm - first) : GM;
    const int in_g = bid - group * GM * tn;
    const int64_t m0 = (int64_t)(first + in_g % gsz) * BM;
    const int64_t n0 = (int64_t)(in_g / gsz) * BN;

    const int nst = (int)(K / BK);
    Panels P;
    P.rowb = (int)(K / 2);
    P.kblocks = (int)(K / 32);
    P.a = panel(A, m0, M, P.rowb);
    P.b = panel(B, n0, N, P.rowb);
    P.sa = panel(SA, m0, M, P.kblocks);
    P.sb = panel(SB, n0, N, P.kblocks);

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // A zero-size twin of the panels: stages past the end of K are "loaded"
    // through it, which returns zeros without touching memory.  Every step
    // then issues exactly one stage of DMA, the number of stages in flight is
    // constant and every wait below is a constant.
    Panels Z = P;
    Z.a = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, 0x00020000);
    Z.b = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, 0, 0x00020000);
    Z.sa = __builtin_amdgcn_make_buffer_rsrc((void*)SA, (short)0, 0, 0x00020000);
    Z.sb = __builtin_amdgcn_make_buffer_rsrc((void*)SB, (short)0, 0, 0x00020000);

#pragma unroll
    for (int p = 0; p < D - 1; p++) stage_dma<BK>(smem + p * G::STAGE, p < nst ? P : Z, p, wave, lane);
    wait_vm<(D - 2) * L>();                          // stage 0 has landed
    bar();
    // two operand sets in ping-pong: X holds even substeps, Y odd ones
    Ops X, Y;
    load_ops<BK>(X, smem, 0, wm, wn, lrow, half);
    static_assert(NSUB == 2, "the loop below is written for two substeps per stage");
    for (int s = 0; s < nst; s++) {
        const uint8_t* st = smem + (s % D) * G::STAGE;
        // substep 0 of stage s, the reads of substep 1 and the DMA of stage
        // s + D - 1 into the buffer of stage s - 1 (every wave finished its
        // reads of it before the previous barrier)
        const int nx = s + D - 1;
        const DmaSlot d = {smem + (nx % D) * G::STAGE, nx < nst ? &P : &Z, nx, wave, lane};
        substep<BK, 0, L>(X, acc, Y, st, 1, wm, wn, lrow, half, &d);
        // stage s + 1 must have landed before its first operands are read
        // (after the last stage the read is of a buffer that is never used)
        wait_vm<(D - 2) * L>();
        bar();
        handover<BK, 1>(smem + ((s + 1) % D) * G::STAGE, Y, acc, X, wm, wn, lrow, half);
    }
    wait_vm<0>();

    if constexpr (CBF16) {
        // stage each wave's 128 x 128 tile as bf16 rows in LDS, then write C
        // with 16-byte stores (each row segment of a wave-store is contiguous)
        __syncthreads();
        uint8_t* ct = smem + wave * 128 * CROW;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    typedef float f2 __attribute__((ext_vector_type(2)));
                    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
                    const f2 f = {acc[i][j][r], acc[i][j][r + 1]};
                    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2));
                    const int ml = i * 32 + 8 * (r / 4) + 4 * half + (r % 4), nl = j * 32 + lrow;
                    *reinterpret_cast<uint16_t*>(ct + ml * CROW + nl * 2) = (uint16_t)w;
                    *reinterpret_cast<uint16_t*>(ct + (ml + 1) * CROW + nl * 2) = (uint16_t)(w >> 16);
                }
        __syncthreads();
        const bool vec = (ldc % 8) == 0;
#pragma unroll 4
        for (int q = 0; q < 32; q++) {
            const int row = q * 4 + (lane >> 4), chunk = lane & 15;
            const int64_t m = m0 + wm * 128 + row, n = n0 + wn * 128 + chunk * 8;
            if (m >= M || n >= N) continue;
            const u32x4v v = *reinterpret_cast<const u32x4v*>(ct + row * CROW + chunk * 16);
            uint16_t* dst = static_cast<uint16_t*>(C) + m * ldc + n;
            if (vec && n + 8 <= N) {
                *reinterpret_cast<u32x4v*>(dst) = v;
            } else {
                const uint32_t e[4] = {v.x, v.y, v.z, v.w};
                for (int k = 0; k < 8 && n + k < N; k++) dst[k] = (uint16_t)(e[k >> 1] >> (16 * (k & 1)));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int64_t n = n0 + wn * 128 + j * 32 + lrow;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                    if (m < M) static_cast<float*>(C)[m * ldc + n] = acc[i][j][r];
                }
            }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c,
                       int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (K % GEMM_BK == 0) {
        const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        if (c_bf16) k_gemm_tiled<true, GEMM_BK, GEMM_D><<<(unsigned)tiles, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
        else k_gemm_tiled<false, GEMM_BK, GEMM_D><<<(unsigned)tiles, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    if (c_bf16) k_gemm_simple<true><<<grid, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
    else k_gemm_simple<false><<<grid, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
    return hipGetLastError();
}

}  // namespace mxk
