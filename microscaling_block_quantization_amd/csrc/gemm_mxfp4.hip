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
#include "gemm_cstore.hpp"

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

// Element formats of the matrix instruction's type fields (CBSZ for A, BLGP for
// B): FP8 E4M3, FP8 E5M2, FP6 E2M3, FP6 E3M2, FP4 E2M1.  The library's own
// element enumeration differs; fmt_of() maps it.
constexpr int MF_E4M3 = 0, MF_E5M2 = 1, MF_E2M3 = 2, MF_E3M2 = 3, MF_E2M1 = 4;
constexpr int fmt_of(int elem) {
    return elem == E2M1 ? MF_E2M1 : elem == E2M3 ? MF_E2M3 : elem == E3M2 ? MF_E3M2 : elem == E4M3 ? MF_E4M3 : MF_E5M2;
}
// bytes of one 32-element block: 16 for E2M1, 24 for FP6, 32 for FP8
constexpr int block_bytes(int mf) { return mf == MF_E2M1 ? 16 : mf >= MF_E2M3 ? 24 : 32; }

// one lane's 4- or 6-bit operand: the 32 codes of one block as the format
// packs them (two E2M1 codes per byte, low nibble first; FP6 as a 6-bit stream
// from the low bit of the first byte), which is the instruction's operand
// layout for those types: four registers for E2M1, six for FP6 (8-bit
// operands: load_fp8_step).  p is 8-byte aligned.
template <int MF>
__device__ __forceinline__ v8i load_block(const uint8_t* p) {
    v8i v;
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0;
    if constexpr (MF == MF_E2M1) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        v[0] = (int)w.x; v[1] = (int)w.y; v[2] = (int)w.z; v[3] = (int)w.w;
    } else {
        const uint2* q = reinterpret_cast<const uint2*>(p);
        const uint2 w0 = q[0], w1 = q[1], w2 = q[2];
        v[0] = (int)w0.x; v[1] = (int)w0.y; v[2] = (int)w1.x; v[3] = (int)w1.y; v[4] = (int)w2.x; v[5] = (int)w2.y;
    }
    return v;
}
// an 8-bit operand of the 64-wide K step that starts at byte `step` of row p:
// the instruction takes K [16h, 16h + 16) of the step in the first four
// registers of the lanes of half h and K [32 + 16h, 48 + 16h) in the last four
// (the scale of half h still covers K [32h, 32h + 32)); a 16-byte piece past
// the end of K (nb blocks in the row) reads as zero
__device__ __forceinline__ v8i load_fp8_step(const uint8_t* p, int64_t step, int half, int64_t nb) {
    v8i v;
    const int64_t b0 = step / 32;                 // the step's first 32-element block
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const bool in = b0 + q < nb;
        const uint4 w = in ? *reinterpret_cast<const uint4*>(p + step + 32 * q + 16 * half) : make_uint4(0, 0, 0, 0);
        v[4 * q] = (int)w.x; v[4 * q + 1] = (int)w.y; v[4 * q + 2] = (int)w.z; v[4 * q + 3] = (int)w.w;
    }
    return v;
}

__device__ __forceinline__ v8i zero_block() {
    v8i v;
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0;
    return v;
}

// Register-only kernel, any element pair: 4 waves of 64 x 64 outputs (2 x 2
// MFMA tiles), operands straight from global memory.
template <bool CBF16, int FA, int FB>
__global__ __launch_bounds__(256) void k_gemm_simple(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                     void* __restrict__ C, int64_t M, int64_t N, int64_t K, int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, row = lane & 31;
    const int64_t m0 = (int64_t)blockIdx.y * TM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * TN + (wave & 1) * 64;
    const int64_t kblocks = K / 32;
    const int64_t rowa = kblocks * block_bytes(FA), rowb = kblocks * block_bytes(FB);

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
        v8i av[2][2], bv[2][2];
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            uint32_t ca[2], cb[2];
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const int64_t kb = k0 / 32 + 2 * kk + half;   // this lane's K block
                const bool in = kb < kblocks;
                const int64_t kb0 = k0 / 32 + 2 * kk;           // the step's first block
                if constexpr (FA == MF_E4M3 || FA == MF_E5M2) av[i][kk] = load_fp8_step(A + ra[i] * rowa, kb0 * 32, half, kblocks);
                else av[i][kk] = in ? load_block<FA>(A + ra[i] * rowa + kb * block_bytes(FA)) : zero_block();
                if constexpr (FB == MF_E4M3 || FB == MF_E5M2) bv[i][kk] = load_fp8_step(B + rb[i] * rowb, kb0 * 32, half, kblocks);
                else bv[i][kk] = in ? load_block<FB>(B + rb[i] * rowb + kb * block_bytes(FB)) : zero_block();
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
                    av[i][0], bv[j][0], acc[i][j], FA, FB, 0, sa[i], 0, sb[j]);
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av[i][1], bv[j][1], acc[i][j], FA, FB, 2, sa[i], 2, sb[j]);
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
// Tiled kernel.  A workgroup of WGM x WGN waves computes a BM x BN output tile
// (BM = WGM * 32 * TI, BN = WGN * 32 * TJ); each wave owns TI x TJ MFMA tiles
// of 32 x 32 (16 fp32 accumulators per lane each).  K advances BK per stage; a
// stage holds the tile's A and B codes (BM and BN rows x BK/2 bytes).  D
// stages form a ring in LDS: stage s + D - 1 is fetched by LDS-DMA
// (buffer_load ... lds, 16 bytes per lane) while stage s is multiplied, so
// every load has D - 1 stages of MFMA work to land.  The 16-byte chunks of a
// code row are XOR-swizzled so that the ds_read_b128 operand reads of
// consecutive rows fall in distinct LDS bank groups.  The E8M0 scales travel
// in groups of SG stages (SG * BK/32 contiguous bytes per row, 16 bytes per
// lane): one scale byte per 16 code bytes would otherwise cost as many L2
// requests as the codes themselves.  Two group buffers alternate in LDS.
// With 8 waves (two per SIMD) one wave's MFMAs run while the other waits on
// its DMA or LDS reads.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int BK_, int WGM_, int WGN_, int TI_, int TJ_>
struct Geo {
    static constexpr int BK = BK_, WGM = WGM_, WGN = WGN_, TI = TI_, TJ = TJ_;
    static constexpr int NW = WGM * WGN;             // waves per workgroup
    static constexpr int BM = WGM * 32 * TI, BN = WGN * 32 * TJ;
    static constexpr int ROWB = BK / 2;              // code bytes per row per stage
    static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPL = 1024 / ROWB;          // rows per 1 KiB wave-load
    static constexpr int SPR = BK / 32;              // scale bytes per row per stage
    static constexpr int ST_A = BM * ROWB, ST_B = BN * ROWB;
    static constexpr int OFF_B = ST_A;
    static constexpr int STAGE = ST_A + ST_B;
    static constexpr int SG = 8;                     // stages per scale group
    static constexpr int SROW = SG * SPR;            // scale bytes per row per group (32)
    static constexpr int SBUF = (BM + BN) * SROW;    // one group: A rows, then B rows
    // wave-loads: code pieces of 1 KiB per stage, scale pieces of 1 KiB per
    // group, dealt evenly to the waves (A's pieces first, then B's)
    static constexpr int LA = ST_A / 1024, LB = ST_B / 1024;
    static constexpr int PWC = (LA + LB) / NW;       // code DMA instructions per wave per stage
    // a scale group is stored as 16-byte units (4 stages of one row) in
    // [half][row] order, A then B: a piece of 64 units covers 64 rows of one half
    static constexpr int LSA = 2 * BM / 64;          // A's scale pieces per group
    static constexpr int PWS = 2 * (BM + BN) / 64 / NW;  // scale DMA instructions per wave per group
    static_assert((LA + LB) % NW == 0 && (2 * (BM + BN) / 64) % NW == 0, "DMA must split evenly over the waves");
    static_assert(SROW == 32 && BM % 64 == 0 && BN % 64 == 0, "two 16-byte units per scale row");
    static_assert(CPR == 4 || CPR == 8, "BK of 128 or 256");
    static constexpr int NOPS = TI + TJ;             // LDS reads per substep (A, then B fragments)
    // physical chunk of logical chunk c in row r (an involution; depends on r mod 16)
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel(const uint8_t* base, int64_t row0, int64_t nrows, int rows,
                                                        int rowbytes) {
    const int64_t valid = nrows - row0 < rows ? nrows - row0 : rows;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * rowbytes), (short)0, (int)(valid * rowbytes),
                                             0x00020000);
}

// DMA instruction k (0 .. L-1) of this wave for stage s into the stage buffer
// `lds`.  Code piece g covers rows [g*RPL, g*RPL + RPL) of its operand; lane l
// writes LDS bytes [16 l, 16 l + 16) of the piece, i.e. row g*RPL + l/CPR at
// physical chunk l%CPR, so it fetches the logical chunk the swizzle stores
// there.  Scale piece h covers 64/DPR rows, one dword per lane.
struct DmaSlot {
    uint8_t* lds;          // uniform LDS destination (goes to M0)
    Panels P;              // the operand panels, or their zero-size twins
    int s, wave, lane;
};

template <class G>
__device__ __forceinline__ void dma_piece(const DmaSlot& d, int k) {
    const int g = d.wave * G::PWC + k;              // uniform
    const bool isb = g >= G::LA;
    const int slot = isb ? g - G::LA : g;
    const int rin = d.lane / G::CPR, pc = d.lane % G::CPR;
    const int row = slot * G::RPL + rin;
    const int vo = rin * d.P.rowb + (G::phys(row, pc) << 4);
    const int so = slot * G::RPL * d.P.rowb + d.s * G::ROWB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isb ? d.P.b : d.P.a,
                                             (lds_void*)(d.lds + (isb ? G::OFF_B : 0) + slot * 1024), 16, vo, so, 0, 0);
}

template <class G>
__device__ __forceinline__ void stage_dma(const DmaSlot& d) {
#pragma unroll
    for (int k = 0; k < G::PWC; k++) dma_piece<G>(d, k);
}

// DMA of scale group `grp` (stages grp*SG ...) into the group buffer `lds`:
// piece h of an operand holds half h/(R/64) of rows 64*(h%(R/64)) + lane
// (R rows), lane l at LDS bytes [16 l, 16 l + 16) of the piece.
template <class G>
__device__ __forceinline__ void scale_dma(uint8_t* lds, __amdgpu_buffer_rsrc_t sa, __amdgpu_buffer_rsrc_t sb,
                                          int kblocks, int grp, int wave, int lane) {
#pragma unroll
    for (int k = 0; k < G::PWS; k++) {
        const int h = wave * G::PWS + k;            // uniform
        const bool isb = h >= G::LSA;
        const int slot = isb ? h - G::LSA : h;
        const int per_half = (isb ? G::BN : G::BM) / 64;
        const int vo = lane * kblocks;
        const int so = (slot % per_half) * 64 * kblocks + grp * G::SROW + (slot / per_half) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isb ? sb : sa,
                                                 (lds_void*)(lds + (isb ? G::BM * G::SROW : 0) + slot * 1024), 16, vo,
                                                 so, 0, 0);
    }
}

// operands of one 64-wide K substep: TI A and TJ B 16-byte fragments
template <class G>
struct Ops {
    u32x4v a[G::TI], b[G::TJ];
};

// the scale bytes of this lane's rows for 4 consecutive stages, read once per
// 4 stages from one 16-byte unit per row tile (4 stages x 4 blocks) and packed
// by a byte permute into two dwords per row tile: p[2c] holds stages 2c and
// 2c+1 as [b(2c, h), b(2c+1, h), b(2c, 2+h), b(2c+1, 2+h)], where b(q, k) is
// block k of stage q and h this lane's half.  Shifted right by 8*(s&1), byte
// 0 is the block of the stage's first substep and byte 2 that of its second
// (the op_sel values 0 and 2).
template <class G>
struct Scl {
    uint32_t p[G::TI + G::TJ][2];
};

template <class G>
__device__ __forceinline__ void load_scl(Scl<G>& o, const uint8_t* __restrict__ buf, int hf, int ra, int rb,
                                         int half) {
    const uint32_t sel = half ? 0x07030501u : 0x06020400u;
    // all reads first, then the permutes: one LDS round trip, not one per row tile
    u32x4v q[G::TI + G::TJ];
#pragma unroll
    for (int i = 0; i < G::TI + G::TJ; i++) {
        const int off = i < G::TI ? (hf * G::BM + ra + 32 * i) * 16
                                  : G::BM * G::SROW + (hf * G::BN + rb + 32 * (i - G::TI)) * 16;
        q[i] = *reinterpret_cast<const u32x4v*>(buf + off);
    }
#pragma unroll
    for (int i = 0; i < G::TI + G::TJ; i++) {
        o.p[i][0] = __builtin_amdgcn_perm(q[i].y, q[i].x, sel);
        o.p[i][1] = __builtin_amdgcn_perm(q[i].w, q[i].z, sel);
    }
}

// this stage's scale operands
template <class G>
struct Cur {
    int x[G::TI + G::TJ];
};

template <class G>
__device__ __forceinline__ void pick(Cur<G>& c, const Scl<G>& sc, int u) {
#pragma unroll
    for (int i = 0; i < G::TI + G::TJ; i++) c.x[i] = (int)((u & 2 ? sc.p[i][1] : sc.p[i][0]) >> (8 * (u & 1)));
}

// LDS read k (0 .. NOPS-1) of the operands of substep t: A fragments, B
// fragments, A scale dwords, B scale dwords.  Rows i*32 apart share the
// swizzle, so the row tiles are immediate offsets from one lane address.
template <class G>
__device__ __forceinline__ void ops_piece(Ops<G>& o, const uint8_t* __restrict__ st, int t, int ra, int rb, int half,
                                          int k) {
    const int c = 2 * t + half;                      // this lane's 32-wide block in the stage
    if (k < G::TI) {
        o.a[k] = *reinterpret_cast<const u32x4v*>(st + ra * G::ROWB + (G::phys(ra, c) << 4) + k * 32 * G::ROWB);
    } else {
        const int j = k - G::TI;
        o.b[j] = *reinterpret_cast<const u32x4v*>(st + G::OFF_B + rb * G::ROWB + (G::phys(rb, c) << 4) +
                                                  j * 32 * G::ROWB);
    }
}

template <class G>
__device__ __forceinline__ void load_ops(Ops<G>& o, const uint8_t* __restrict__ st, int t, int ra, int rb, int half) {
#pragma unroll
    for (int k = 0; k < G::NOPS; k++) ops_piece<G>(o, st, t, ra, rb, half, k);
}

// One substep in a fixed instruction order: MFMA k of `cur`, then its share of
// the LDS reads of the next operands and of the DMA of a later stage, with a
// scheduling fence after each step.  A DMA instruction holds the wave at the
// texture unit for a while and the MFMA in flight hides it; every LDS read
// has the rest of the substep to land.  After the shift by 8*half this lane's
// scale byte (block 2t + half of the stage) is byte 2*(t&1): the op_sel value.
template <class G, int T1, int NV, int NOFF>
__device__ __forceinline__ void substep(const Ops<G>& cur, const Cur<G>& sc, v16f (&acc)[G::TI][G::TJ], Ops<G>& nxt,
                                        const uint8_t* __restrict__ st, int t, int ra, int rb, int half,
                                        const DmaSlot* d) {
    constexpr int NM = G::TI * G::TJ;
    int xa[G::TI], xb[G::TJ];
#pragma unroll
    for (int i = 0; i < G::TI; i++) xa[i] = sc.x[i];
#pragma unroll
    for (int j = 0; j < G::TJ; j++) xb[j] = sc.x[G::TI + j];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NM; k++) {
        const int i = k / G::TJ, j = k % G::TJ;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8(cur.a[i]), op8(cur.b[j]), acc[i][j], 4, 4,
                                                                   2 * T1, xa[i], 2 * T1, xb[j]);
        // An empty volatile statement that names the result: it emits nothing,
        // but it keeps the MFMA ahead of the fence below.  (The result is only
        // used by the next stage, so the instruction selector would otherwise
        // place every MFMA of the substep after the last fence.)
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" ::"v"(acc[i][j]));
#endif
#pragma unroll
        for (int q = k * G::NOPS / NM; q < (k + 1) * G::NOPS / NM; q++) ops_piece<G>(nxt, st, t, ra, rb, half, q);
        // the NV DMA pieces spread evenly, half a spacing in: with 4 pieces
        // over 8 MFMAs, after MFMAs 1, 3, 5 and 7
#pragma unroll
        for (int q = 0; q < NV; q++)
            if (q * NM / NV + NM / (2 * NV) == k) dma_piece<G>(*d, NOFF + q);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// wait until at most N vector-memory ops of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// the same with N0, N1 or N2 chosen by a uniform sel (0, 1, 2).  One asm
// statement: a branch in the source would split the basic block, and the
// compiler then sinks the preceding MFMAs below the wait.
template <int N0, int N1, int N2>
__device__ __forceinline__ void wait_vm_sel(int sel) {
    asm volatile(
        "s_cmp_eq_u32 %0, 0\n\t"
        "s_cbranch_scc1 1f\n\t"
        "s_cmp_eq_u32 %0, 1\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_waitcnt vmcnt(%3)\n\t"
        "s_branch 3f\n"
        "1:\n\t"
        "s_waitcnt vmcnt(%1)\n\t"
        "s_branch 3f\n"
        "2:\n\t"
        "s_waitcnt vmcnt(%2)\n"
        "3:" ::"s"(sel), "n"(N0), "n"(N1), "n"(N2) : "memory", "scc");
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

// the stage handover: the last substep of the current stage multiplies while
// the first operands of the next stage are read from `nxt`.  It issues no DMA:
// a whole stage goes out in the substep after it (measured 2-4% faster than
// half of it here, half there).  The buffers are distinct restrict-qualified
// objects, so the operand reads carry no dependence on the DMA in flight.
template <class G, int T1>
__device__ __forceinline__ void handover(const uint8_t* __restrict__ nxt, const Ops<G>& cur, const Cur<G>& sc,
                                         v16f (&acc)[G::TI][G::TJ], Ops<G>& o, int ra, int rb, int half) {
    substep<G, T1, 0, 0>(cur, sc, acc, o, nxt, 0, ra, rb, half, nullptr);
}

template <bool CBF16, bool EXACT, class G, int D>
__global__ __launch_bounds__(64 * G::NW, 1) void k_gemm_tiled(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ SA,
                                                              const uint8_t* __restrict__ B,
                                                              const uint8_t* __restrict__ SB, void* __restrict__ C,
                                                              int64_t M, int64_t N, int64_t K, int64_t ldc) {
    static_assert(D >= 3 && D <= 4, "ring depth: the handover waits for the next stage while D - 3 more are in flight");
    static_assert(G::BK == 128, "the loop below is written for two substeps per stage");
    constexpr int TI = G::TI, TJ = G::TJ, L = G::PWC, SG = G::SG;
    using CS = CStore<G>;
    constexpr int NSTORE = CS::NSTORE;
    static_assert(SG > 2 * D - 4, "no scale group opens among the stages that overlap the previous tile's stores");
    static_assert((D - 2) * L + G::PWS <= 63 && (D - 2) * L + NSTORE <= 63, "vector-memory wait counts fit vmcnt");
    static_assert(G::NW * CS::AREA <= G::STAGE, "C strips are staged in the last ring slot");
    // the code ring, then the two scale-group buffers
    __shared__ __attribute__((aligned(16))) uint8_t smem[D * G::STAGE + 2 * G::SBUF];
    uint8_t* const sgb = smem + D * G::STAGE;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, lrow = lane & 31;
    const int wm = wave / G::WGN, wn = wave % G::WGN;
    const int ra = wm * 32 * TI + lrow, rb = wn * 32 * TJ + lrow;   // this lane's operand rows in the tile
    uint8_t* const ct = smem + (D - 1) * G::STAGE + wave * CS::AREA;

    // XCD-aware, grouped tile order: workgroup slots are dealt to the 8 XCDs
    // round robin, so consecutive tiles of the grouped order go to one XCD and
    // share A and B panels in its L2.  The workgroups are persistent: slot
    // blockIdx.x + k * gridDim.x is a workgroup's k-th tile.
    const int tm = (int)((M + G::BM - 1) / G::BM), tn = (int)((N + G::BN - 1) / G::BN);
    const int T = tm * tn;
    auto tile_of = [&](int lin, int64_t& m0, int64_t& n0) {
        int bid = lin;
        if (T % 8 == 0) bid = (bid % 8) * (T / 8) + bid / 8;
        constexpr int GM = 8;
        const int group = bid / (GM * tn);
        const int first = group * GM;
        const int gsz = (tm - first) < GM ? (tm - first) : GM;
        const int in_g = bid - group * GM * tn;
        m0 = (int64_t)(first + in_g % gsz) * G::BM;
        n0 = (int64_t)(in_g / gsz) * G::BN;
    };
    const int nst = (int)(K / G::BK);
    const int rowb = (int)(K / 2), kblocks = (int)(K / 32);
    auto panels_of = [&](int64_t m0, int64_t n0) {
        Panels P;
        P.rowb = rowb;
        P.kblocks = kblocks;
        P.a = panel(A, m0, M, G::BM, rowb);
        P.b = panel(B, n0, N, G::BN, rowb);
        P.sa = panel(SA, m0, M, G::BM, kblocks);
        P.sb = panel(SB, n0, N, G::BN, kblocks);
        return P;
    };
    // A zero-size twin of the panels: stages past the end of K are "loaded"
    // through it, which returns zeros without touching memory.  Every step
    // then issues exactly one stage of DMA, the number of stages in flight is
    // constant and every wait below is a constant.
    Panels Z;
    Z.rowb = rowb;
    Z.kblocks = kblocks;
    Z.a = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, 0x00020000);
    Z.b = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, 0, 0x00020000);
    Z.sa = __builtin_amdgcn_make_buffer_rsrc((void*)SA, (short)0, 0, 0x00020000);
    Z.sb = __builtin_amdgcn_make_buffer_rsrc((void*)SB, (short)0, 0, 0x00020000);
    // the first D - 1 stages of a tile: scale group 0 goes first, ahead of the
    // codes of stage 0, so waiting for a stage's codes also covers its scales
    // (vector memory completes in order)
    auto prologue = [&](const Panels& P) {
        scale_dma<G>(sgb, P.sa, P.sb, P.kblocks, 0, wave, lane);
#pragma unroll
        for (int p = 0; p < D - 1; p++) {
            const DmaSlot d = {smem + p * G::STAGE, p < nst ? P : Z, p, wave, lane};
            stage_dma<G>(d);
        }
    };
    // EXACT (bf16 C, ldc and N multiples of 8): stores of whole 16-byte
    // chunks, an exact count per wave
    static_assert(!EXACT || CBF16, "the exact store path writes bf16");
    constexpr bool exact = EXACT;

    int lin = blockIdx.x;
    int64_t m0, n0;
    tile_of(lin, m0, n0);
    Panels P = panels_of(m0, n0);

    v16f acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // a stage's codes go out in the first substep after the barrier that
    // frees its slot; the scale group that stage st_ opens, if any, goes out
    // right after that barrier, ahead of them
    auto open_group = [&](const Panels& P_, int st_) {
        if (st_ % SG == 0)
            scale_dma<G>(sgb + ((st_ / SG) & 1) * G::SBUF, st_ < nst ? P_.sa : Z.sa, st_ < nst ? P_.sb : Z.sb,
                         P_.kblocks, st_ / SG, wave, lane);
    };
    prologue(P);
    wait_vm<(D - 2) * L>();                          // stage 0 and scale group 0 have landed
    bar();
    open_group(P, D - 1);
    // two operand sets in ping-pong: X holds even substeps, Y odd ones; the
    // scale registers hold 4 stages and are refilled at every 4th stage
    Ops<G> X, Y;
    Scl<G> S;
    Cur<G> Q;
    load_ops<G>(X, smem, 0, ra, rb, half);
    load_scl<G>(S, sgb, 0, ra, rb, half);
    bool pend = false;       // the previous tile's C stores are in flight, issued after this tile's first stages
    for (;;) {
        for (int s = 0; s < nst; s++) {
            const uint8_t* st = smem + (s % D) * G::STAGE;
            // stages 0 .. 3 of a tile were read after its first stage landed
            if ((s & 3) == 0 && s > 0) load_scl<G>(S, sgb + ((s / SG) & 1) * G::SBUF, (s % SG) / 4, ra, rb, half);
            pick<G>(Q, S, s & 3);
            // substep 0 of stage s, the reads of substep 1 and the DMA of stage
            // s + D - 1 (into the slot the barrier before freed)
            const int nx = s + D - 1;
            const DmaSlot d = {smem + (nx % D) * G::STAGE, nx < nst ? P : Z, nx, wave, lane};
            substep<G, 0, L, 0>(X, Q, acc, Y, st, 1, ra, rb, half, &d);
            // stage s + 1 (and its scales) must have landed before its first
            // operands are read.  What may stay in flight: the DMA of the
            // later stages, one scale group if one of them opens a group, and
            // the previous tile's C stores while they are younger than stage
            // s + 1 (after the last stage the read is of a buffer never used).
            bool extra = false;
#pragma unroll
            for (int q = 2; q <= D - 1; q++) extra = extra || ((s + q) % SG == 0);
            const int sel = (pend && s < D - 2) ? 2 : (extra ? 1 : 0);
            wait_vm_sel<(D - 2) * L, (D - 2) * L + G::PWS, (D - 2) * L + NSTORE>(
                __builtin_amdgcn_readfirstlane(sel));
            bar();
            // slot s % D is free now for stage s + D, whose codes go out in the
            // next substep; its scale group, if it opens one, goes out here
            open_group(P, s + D);
            handover<G, 1>(smem + ((s + 1) % D) * G::STAGE, Y, Q, acc, X, ra, rb, half);
        }
        wait_vm<0>();        // this tile's DMA, including the zero-size loads past K
        bar();               // every wave is done with the ring and the scale buffers

        const int nlin = lin + (int)gridDim.x;
        const bool more = nlin < T;
        int64_t nm0 = 0, nn0 = 0;
        Panels NP = P;
        if (more) {
            tile_of(nlin, nm0, nn0);
            NP = panels_of(nm0, nn0);
        }
        if constexpr (exact) {
            // the next tile's first stages go out first; the stores follow and
            // drain while that tile starts
            if (more) prologue(NP);
            store_c_bf16<G, true>(acc, ct, C, m0, n0, M, N, ldc, wm, wn, lane, half, lrow);
        } else {
            if constexpr (CBF16) {
                store_c_bf16<G, false>(acc, ct, C, m0, n0, M, N, ldc, wm, wn, lane, half, lrow);
            } else {
#pragma unroll
                for (int i = 0; i < TI; i++)
#pragma unroll
                    for (int j = 0; j < TJ; j++) {
                        const int64_t n = n0 + wn * 32 * TJ + j * 32 + lrow;
                        if (n >= N) continue;
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            const int64_t m = m0 + wm * 32 * TI + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                            if (m < M) static_cast<float*>(C)[m * ldc + n] = acc[i][j][r];
                        }
                    }
            }
            wait_vm<0>();
            if (more) prologue(NP);
        }
        if (!more) break;
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < TJ; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
        // the next tile's stage 0 and scale group 0 must have landed; its
        // stages 1 .. D-2 and, on the exact path, the C stores may stay in flight
        if constexpr (exact) wait_vm<(D - 2) * L + NSTORE>();
        else wait_vm<(D - 2) * L>();
        bar();               // also: every wave's strip reads are done before stage D-1's DMA refills that slot
        open_group(NP, D - 1);
        load_ops<G>(X, smem, 0, ra, rb, half);
        load_scl<G>(S, sgb, 0, ra, rb, half);
        lin = nlin;
        m0 = nm0;
        n0 = nn0;
        P = NP;
        pend = exact;
    }
}

#ifndef GEMM_WAVES
#define GEMM_WAVES 8
#endif
// 4 waves: 2 x 2 waves of 4 x 4 MFMA tiles; 8 waves: 2 x 4 waves of 4 x 2
using GemmGeo = Geo<GEMM_BK, 2, GEMM_WAVES / 2, 4, GEMM_WAVES == 8 ? 2 : 4>;

template <int FA, int FB>
void launch_simple(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c,
                   int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    if (c_bf16) k_gemm_simple<true, FA, FB><<<grid, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
    else k_gemm_simple<false, FA, FB><<<grid, 256, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
}

template <int FA>
void launch_simple_b(int eb, const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c,
                     int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    switch (fmt_of(eb)) {
    case MF_E2M1: launch_simple<FA, MF_E2M1>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    case MF_E2M3: launch_simple<FA, MF_E2M3>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    case MF_E3M2: launch_simple<FA, MF_E3M2>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    case MF_E4M3: launch_simple<FA, MF_E4M3>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    default: launch_simple<FA, MF_E5M2>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    }
}

}  // namespace

bool gemm_elem_ok(int elem) { return elem == E2M1 || elem == E2M3 || elem == E3M2 || elem == E4M3 || elem == E5M2; }

hipError_t launch_gemm(int ea, const uint8_t* a, const uint8_t* sa, int eb, const uint8_t* b, const uint8_t* sb,
                       void* c, int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s,
                       const uint8_t* ma, const uint8_t* mb) {
    if (M == 0 || N == 0) return hipSuccess;
    if (!gemm_elem_ok(ea) || !gemm_elem_ok(eb)) return hipErrorInvalidValue;
    if (ma || mb) {
        // macro-block scaled MXFP4 (K is a multiple of 128 with macro blocks)
        if (ea != E2M1 || eb != E2M1 || K % 128) return hipErrorInvalidValue;
        return launch_gemm_lds(ea, a, sa, eb, b, sb, c, M, N, K, ldc, c_bf16, s, ma, mb);
    }
    // the tiled kernel (E2M1 operands) fetches scales in 32-byte row groups (8
    // stages of 128): with K a multiple of 1024 every scale row starts 32-byte
    // aligned
    if (ea == E2M1 && eb == E2M1 && K % 1024 == 0) {
        using G = GemmGeo;
        const int64_t tiles = ((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN);
        // persistent: one workgroup per CU (the LDS ring fills a CU), each
        // looping over its tiles
        static int cus = 0;
        if (cus == 0) {
            int dev = 0, c = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
                cus = c;
            else
                cus = 256;
        }
        const int64_t grid = tiles < cus ? tiles : cus;
        const bool exact = c_bf16 && ldc % 8 == 0 && N % 8 == 0 && (int64_t)G::BM * ldc * 2 < 0x80000000LL;
        if (exact)
            k_gemm_tiled<true, true, G, GEMM_D><<<(unsigned)grid, 64 * G::NW, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
        else if (c_bf16)
            k_gemm_tiled<true, false, G, GEMM_D><<<(unsigned)grid, 64 * G::NW, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
        else
            k_gemm_tiled<false, false, G, GEMM_D><<<(unsigned)grid, 64 * G::NW, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc);
        return hipGetLastError();
    }
    // K a multiple of 128: the LDS-staged kernel for any element pair
    if (K % 128 == 0) return launch_gemm_lds(ea, a, sa, eb, b, sb, c, M, N, K, ldc, c_bf16, s);
    switch (fmt_of(ea)) {
    case MF_E2M1: launch_simple_b<MF_E2M1>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    case MF_E2M3: launch_simple_b<MF_E2M3>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    case MF_E3M2: launch_simple_b<MF_E3M2>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    case MF_E4M3: launch_simple_b<MF_E4M3>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    default: launch_simple_b<MF_E5M2>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s); break;
    }
    return hipGetLastError();
}

}  // namespace mxk
