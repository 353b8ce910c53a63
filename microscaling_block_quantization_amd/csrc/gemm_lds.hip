// gemm_lds.hip -- LDS-staged block-scaled GEMM for MXFP8, MXFP6 and mixed
// 8-/6-/4-bit operands: C = deq(A) . deq(B)^T with E8M0 scales per 1 x 32
// block and each operand's elements E2M1, E2M3, E3M2, E4M3 or E5M2, on
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 (the 6-bit and mixed products of the ARITH
// 2025 MX-training report, main results; MX also has 8-bit elements,
// "Unveiling the Potential of Quantization with MXFP4", current state).
//
// A workgroup of 8 waves (2 x 4) computes a 256 x 256 tile; each wave owns 4 x 2
// MFMA tiles of 32 x 32.  K advances 128 per stage (two 64-wide substeps); a
// stage holds the tile's A and B codes, 64 bytes per row for E2M1, 96 for FP6
// and 128 for FP8 (pairs with 8-bit operands use 128 x 256 or 256 x 128
// tiles, or 256 x 256 with E2M1, so that three stages fit in LDS).  Three stages form a ring in LDS, filled by LDS-DMA (buffer_load ...
// lds, 16 bytes per lane) two stages ahead.  The 16-byte chunks of a row are
// permuted by a row-dependent rotation (FP6) or XOR (E2M1, FP8) so that the
// chunk reads of 16 consecutive rows fall in distinct LDS banks.  An FP6
// operand (32 codes, 24 bytes) spans one whole chunk and half of the next: two
// 16-byte reads, put in order per lane; an FP8 operand is two whole chunks.  The block scales (4 bytes per row and stage)
// come by LDS-DMA too, in groups of 4 stages (16 bytes of a row per lane: a
// quarter of the L2 requests of a dword per stage), so that the only loads in
// flight in the loop are the DMA the stage waits count (and, with macro-block
// scales, one byte per operand row a stage ahead).
#include "mx_kernels.hpp"
#include "gemm_cstore.hpp"

namespace mxk {
using namespace mxd;

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// the instruction's type codes: FP8 E4M3 0, E5M2 1, FP6 E2M3 2, E3M2 3, FP4 E2M1 4
constexpr int MF_E2M1 = 4;
constexpr int lmf(int elem) { return elem == E2M1 ? 4 : elem == E2M3 ? 2 : elem == E3M2 ? 3 : elem == E4M3 ? 0 : 1; }
constexpr bool is_fp8(int f) { return f <= 1; }
// bytes of one 32-element block
constexpr int lbb(int f) { return f == MF_E2M1 ? 16 : is_fp8(f) ? 32 : 24; }

template <int F>
struct Op {
    static constexpr int R = 4 * lbb(F);               // bytes per row per stage
    static constexpr int C = R / 16;                   // chunks per row
    // physical chunk slot of logical chunk p in tile row r, and back
    // FP6: a rotation by one slot in row quads 1 and 2 of every 16 rows; the
    // 16-byte reads of one logical chunk by 16 consecutive rows then cover 64
    // distinct banks (and those of 8 rows 32 banks)
    static __device__ __forceinline__ int rot(int r) { return ((r >> 2) & 1) ^ ((r >> 3) & 1); }
    // FP8: 8 chunks per row, XOR by the row's low 3 bits (the 8 rows of one
    // phase of a 16-byte read fall on 8 distinct chunk slots)
    static __device__ __forceinline__ int phys(int r, int p) {
        if constexpr (C == 4) return p ^ (((r >> 1) & 3) ^ ((r >> 3) & 1));
        else if constexpr (C == 8) return p ^ (r & 7);
        else return (p + rot(r)) % 6;
    }
    static __device__ __forceinline__ int logical(int r, int q) {
        if constexpr (C == 4) return q ^ (((r >> 1) & 3) ^ ((r >> 3) & 1));
        else if constexpr (C == 8) return q ^ (r & 7);
        else return (q + 6 - rot(r)) % 6;
    }
};

template <int FA_, int FB_, int WGM_, int WGN_, int TI_, int TJ_, int MBS_ = 0, int SG_ = 4>
struct LGeo {
    static constexpr int FA = FA_, FB = FB_, MBS = MBS_;
    static constexpr int WGM = WGM_, WGN = WGN_, TI = TI_, TJ = TJ_;   // waves, MFMA tiles per wave
    static constexpr int NW = WGM * WGN, BM = WGM * 32 * TI, BN = WGN * 32 * TJ, BK = 128, D = 3;
    static constexpr int SA = BM * Op<FA_>::R, SB = BN * Op<FB_>::R;
    // macro-block scales (MBS bit 0: A, bit 1: B; a stage is one 128-wide
    // macro block): each lane loads the bytes of its operand rows with the
    // stage's E8M0 scales; A's go through LDS, decoded to fp32 (4 BM bytes
    // after the codes), to the lanes that hold those rows' accumulators
    static constexpr int NS = MBS ? TI + TJ : 1;       // macro scale registers per stage
    static constexpr int OFF_M = SA + SB;
    static constexpr int STAGE = OFF_M + ((MBS & 1) ? 4 * BM : 0);
    static constexpr int PA = SA / 1024, PB = SB / 1024;
    static constexpr int PW = (PA + PB) / NW;          // code DMA pieces per wave per stage
    // block scales travel in groups of SG stages, the 4 SG bytes of a row per
    // lane, into NB buffers after the ring: groups of 4 stages (K >= 512) one
    // group ahead in two buffers, or single stages two ahead in three
    static constexpr int SG = SG_;
    static constexpr int NB = SG == 1 ? 3 : 2;
    static constexpr int GROW = 4 * SG;
    static constexpr int GBUF = (BM + BN) * GROW;
    static constexpr int OFF_G = D * STAGE;
    // group DMA: (BM + BN) / 64 pieces of 64 rows, GPW per wave; when they do
    // not split evenly, the waves past the last piece load through the
    // zero-size resource into a 1 KiB sink, so that every wave issues the
    // same count (the stage waits count them)
    static constexpr int GP = (BM + BN) / 64;
    static constexpr int GPW = (GP + NW - 1) / NW;
    static constexpr int OFF_SINK = OFF_G + NB * GBUF;
    static constexpr int SMEM = OFF_SINK + (GP % NW ? 1024 : 0);
    static_assert(SG == 1 || SG == 4, "scale groups of 1 or 4 stages");
    static_assert((PA + PB) % NW == 0 && (BM + BN) % 64 == 0, "code DMA pieces split evenly over the waves");
    static_assert(GPW == 1 || (BM / 64) % GPW == 0, "a wave's scale pieces lie in one operand");
};

__device__ __forceinline__ rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// one lane's operand for K block c (0..3) of the stage, tile row rr, from the
// stage region `st` of its operand
template <int F>
__device__ __forceinline__ v8i frag(const uint8_t* __restrict__ st, int rr, int t, int half) {
    using O = Op<F>;
    v8i v;
    if constexpr (is_fp8(F)) {
        // 8-bit operands are split by the instruction: the lanes of half h
        // supply K [16h, 16h + 16) of the 64-wide step in their first four
        // registers and K [32 + 16h, 48 + 16h) in the last four (the scale of
        // half h still covers K [32h, 32h + 32)): chunks 4t + h and 4t + 2 + h
        const int c = 4 * t + half;
        const u32x4v x = *reinterpret_cast<const u32x4v*>(st + rr * O::R + O::phys(rr, c) * 16);
        const u32x4v y = *reinterpret_cast<const u32x4v*>(st + rr * O::R + O::phys(rr, c + 2) * 16);
        v[0] = (int)x[0]; v[1] = (int)x[1]; v[2] = (int)x[2]; v[3] = (int)x[3];
        v[4] = (int)y[0]; v[5] = (int)y[1]; v[6] = (int)y[2]; v[7] = (int)y[3];
        return v;
    } else if constexpr (F == MF_E2M1) {
        const u32x4v x = *reinterpret_cast<const u32x4v*>(st + rr * O::R + O::phys(rr, 2 * t + half) * 16);
        v[0] = (int)x[0]; v[1] = (int)x[1]; v[2] = (int)x[2]; v[3] = (int)x[3];
        v[4] = 0; v[5] = 0;
    } else {
        // block 2t + h covers bytes [48t + 24h, +24): the whole chunk 3t + 2h
        // and half h of chunk 3t + 1.  Both halves read all of chunk 3t + 1
        // (one logical chunk per read, so the rotation keeps it free of bank
        // conflicts); half 0 puts its first 8 bytes after the whole chunk,
        // half 1 its last 8 bytes before it
        const u32x4v x = *reinterpret_cast<const u32x4v*>(st + rr * O::R + O::phys(rr, 3 * t + 2 * half) * 16);
        const u32x4v y = *reinterpret_cast<const u32x4v*>(st + rr * O::R + O::phys(rr, 3 * t + 1) * 16);
        v[0] = (int)(half ? y[2] : x[0]);
        v[1] = (int)(half ? y[3] : x[1]);
        v[2] = (int)(half ? x[0] : x[2]);
        v[3] = (int)(half ? x[1] : x[3]);
        v[4] = (int)(half ? x[2] : y[0]);
        v[5] = (int)(half ? x[3] : y[1]);
    }
    v[6] = 0;
    v[7] = 0;
    return v;
}

// substep T of a stage: K blocks 2T (lanes of half 0) and 2T + 1 (half 1);
// this lane's scale byte is byte 2T of sc after the shift by 8 * half
template <int T, class G>
__device__ __forceinline__ void substep(v16f (&acc)[G::TI][G::TJ], const uint8_t* __restrict__ st, int ra, int rb,
                                        int half, const int (&sc)[G::TI + G::TJ]) {
    v8i a[G::TI], b[G::TJ];
#pragma unroll
    for (int i = 0; i < G::TI; i++) a[i] = frag<G::FA>(st, ra + 32 * i, T, half);
#pragma unroll
    for (int j = 0; j < G::TJ; j++) b[j] = frag<G::FB>(st + G::SA, rb + 32 * j, T, half);
#pragma unroll
    for (int i = 0; i < G::TI; i++)
#pragma unroll
        for (int j = 0; j < G::TJ; j++)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], G::FA, G::FB, 2 * T,
                                                                       sc[i], 2 * T, sc[G::TI + j]);
}

// (MBS) one stage's product folded into the totals tile by tile: the stage's
// two substeps go into a fresh accumulator (a zero C operand), which is then
// added to the total times s_M^A of each accumulator row and s_M^B of its
// column; that product of two UE4M3 values is exact in fp32.  The next tile's
// products are issued before this tile's fold, so the fold does not wait on
// the matrix unit; two fresh tiles are live.
template <class G>
__device__ __forceinline__ void mbs_stage(v16f (&acc)[G::TI][G::TJ], const uint8_t* __restrict__ st, int ra, int rb,
                                          int half, const int (&sc)[G::TI + G::TJ], const float (&fb)[G::TJ]) {
    constexpr int NTL = G::TI * G::TJ;
    v8i b0[G::TJ], b1[G::TJ];
#pragma unroll
    for (int j = 0; j < G::TJ; j++) {
        b0[j] = frag<G::FB>(st + G::SA, rb + 32 * j, 0, half);
        b1[j] = frag<G::FB>(st + G::SA, rb + 32 * j, 1, half);
    }
    const float* ms = reinterpret_cast<const float*>(st + G::OFF_M);
    // accumulator register 4q + p holds row 8q + 4 half + p of the tile
    const int r0 = ra - (ra & 31) + 4 * half;
    v8i a0 = frag<G::FA>(st, ra, 0, half), a1 = frag<G::FA>(st, ra, 1, half);
    auto product = [&](int k) -> v16f {
        const int i = k / G::TJ, j = k % G::TJ;
        const v16f t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0[j], v16f{}, G::FA, G::FB, 0, sc[i], 0,
                                                                       sc[G::TI + j]);
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1[j], t, G::FA, G::FB, 2, sc[i], 2,
                                                               sc[G::TI + j]);
    };
    v16f tc = product(0);
#pragma unroll
    for (int k = 0; k < NTL; k++) {
        const int i = k / G::TJ, j = k % G::TJ;
        v16f tn;
        if (k + 1 < NTL) {
            if ((k + 1) % G::TJ == 0) {
                a0 = frag<G::FA>(st, ra + 32 * ((k + 1) / G::TJ), 0, half);
                a1 = frag<G::FA>(st, ra + 32 * ((k + 1) / G::TJ), 1, half);
            }
            tn = product(k + 1);
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            v4f w = {1.f, 1.f, 1.f, 1.f};
            if constexpr ((G::MBS & 1) != 0) w = *reinterpret_cast<const v4f*>(ms + r0 + 32 * i + 8 * q);
#pragma unroll
            for (int pp = 0; pp < 4; pp++)
                acc[i][j][4 * q + pp] = __builtin_fmaf(tc[4 * q + pp], w[pp] * fb[j], acc[i][j][4 * q + pp]);
        }
        if (k + 1 < NTL) tc = tn;
    }
}

// the operand panels of one tile: rows past M (N) read as zero through the
// resource bounds; z is a zero-size resource for stages past K
struct LPanels {
    rsrc_t a, b, sa, sb, z, ma, mb;
    int64_t rowa, rowb;
    int kblocks, nst, mcols;
};

// DMA of stage s into its ring slot; stages past K go through the zero-size
// resource (no memory access), so every stage issues the same count.  Piece g
// of the codes covers 64 consecutive 16-byte LDS slots; the lane writing slot
// (row r, physical chunk q) fetches the logical chunk stored there.  Then the
// stage's scale dword of each tile row.  The operand of a piece is a select,
// not a branch: with no branch around the loads the compiler's own counts of
// loads in flight stay exact, and it never waits for a stage still in flight.
template <class G>
__device__ __forceinline__ void stage_dma(uint8_t* smem, const LPanels& P, int s, int wave, int lane) {

    // (device pass only: the host pass of this template rejects the LDS-DMA
    // builtin, which would silently drop the kernels' launch stubs)
#if defined(__HIP_DEVICE_COMPILE__)
    using OA = Op<G::FA>;
    using OB = Op<G::FB>;
    uint8_t* slot = smem + (s % G::D) * G::STAGE;
    const bool in = s < P.nst;
    const rsrc_t pa = P.a, pb = P.b, pz = P.z;
    const int rowa = (int)P.rowa, rowb = (int)P.rowb;
#pragma unroll
    for (int k = 0; k < G::PW; k++) {
        const int g = wave * G::PW + k;                   // uniform
        const bool isb = g >= G::PA;
        const int f = (isb ? g - G::PA : g) * 64 + lane;
        const int ra = f / OA::C, rb = f / OB::C;
        const int va = ra * rowa + OA::logical(ra, f % OA::C) * 16;
        const int vb = rb * rowb + OB::logical(rb, f % OB::C) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(in ? (isb ? pb : pa) : pz, (lds_void*)(slot + g * 1024), 16,
                                                 isb ? vb : va, s * (isb ? OB::R : OA::R), 0, 0);
    }
#endif
}

// first scale byte of group g that its buffer holds: groups of 4 stages
// start 16 g into the row, except a partial last group, which is read as the
// row's last 16 bytes so that no load reaches past the row (the panel's last
// row ends at the resource bound)
template <class G>
__device__ __forceinline__ int group_start(int g, int kblocks) {
    if constexpr (G::SG == 1) return 4 * g;
    else return 16 * g < kblocks - 16 ? 16 * g : kblocks - 16;
}

// DMA of scale group g (stages SG g .. SG g + SG - 1) into its buffer: one
// row's 4 SG bytes per lane.  Groups past K read through the zero-size
// resource.
template <class G>
__device__ __forceinline__ void group_dma(uint8_t* smem, const LPanels& P, int g, int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    const rsrc_t psa = P.sa, psb = P.sb, pz = P.z;
    const bool in = g * G::SG < P.nst;
    uint8_t* buf = smem + G::OFF_G + (g % G::NB) * G::GBUF;
    const int start = group_start<G>(g, P.kblocks);
#pragma unroll
    for (int k = 0; k < G::GPW; k++) {
        const int q = wave * G::GPW + k;                  // uniform
        const bool real = q < G::GP;
        const bool isb = q >= G::BM / 64;
        const int row = (isb ? q - G::BM / 64 : q) * 64 + lane;
        uint8_t* dst = real ? buf + q * 64 * G::GROW : smem + G::OFF_SINK;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(in && real ? (isb ? psb : psa) : pz, (lds_void*)dst, G::GROW,
                                                 row * P.kblocks + start, 0, 0, 0);
    }
#endif
}

// (MBS) the macro scale byte of stage s of each of this lane's operand rows
// (A: TI, then B: TJ), a stage ahead
template <class G>
__device__ __forceinline__ void stage_macro(uint32_t (&o)[G::NS], const LPanels& P, int s, int ra, int rb) {
    if constexpr (G::MBS != 0) {
        const bool in = s < P.nst;
        const rsrc_t pma = P.ma, pmb = P.mb, pz = P.z;
#pragma unroll
        for (int i = 0; i < G::TI; i++)
            o[i] = (G::MBS & 1) ? __builtin_amdgcn_raw_buffer_load_b8(in ? pma : pz, (ra + 32 * i) * P.mcols + s, 0, 0)
                                : 0x38u;
#pragma unroll
        for (int j = 0; j < G::TJ; j++)
            o[G::TI + j] = (G::MBS & 2) ? __builtin_amdgcn_raw_buffer_load_b8(in ? pmb : pz, (rb + 32 * j) * P.mcols + s, 0, 0)
                                        : 0x38u;
    }
}

// value of a UE4M3 macro-block scale code (E4M3 bits, bias 7, sign clear)
__device__ __forceinline__ float ue4m3(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// a bare workgroup barrier after this wave's LDS reads are done (the DMA the
// barrier publishes was waited for with wait_vm)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// one stage: wait for its DMA (codes and scales), free the slot two ahead,
// issue the next stage's macro scales and the DMA two stages ahead, multiply
template <class G>
__device__ __forceinline__ void lds_step(uint8_t* smem, const LPanels& P, int s, int wave, int lane, int half, int ra,
                                         int rb, v16f (&acc)[G::TI][G::TJ], const uint32_t (&cur)[G::NS],
                                         uint32_t (&nxt)[G::NS]) {
    // in flight after stage s's codes: the codes of s + 1, and a scale group
    // if stage s - 1 issued one after them (every stage with single-stage
    // groups, whose prologue issues groups 0 and 1 in the same order)
    if (G::SG == 1 || (s & (G::SG - 1)) == 1) wait_vm<G::PW + G::GPW>();
    else wait_vm<G::PW>();
    if constexpr ((G::MBS & 1) != 0) {
        // A's macro scales of stage s, decoded, to LDS for the accumulator
        // rows (waves that share A rows write the same values)
        float* ms = reinterpret_cast<float*>(smem + (s % G::D) * G::STAGE + G::OFF_M);
#pragma unroll
        for (int i = 0; i < G::TI; i++) ms[ra + 32 * i] = ue4m3(cur[i]);
    }
    // every wave's share of stage s has landed and every wave is done
    // reading slot (s + 2) % 3 (stage s - 1)
    lds_barrier();
    stage_macro<G>(nxt, P, s + 1, ra, rb);
    stage_dma<G>(smem, P, s + 2, wave, lane);
    // the next scale group into the buffer of a group every wave has finished
    // reading (before the barrier above): 4-stage groups one ahead, single
    // stages two ahead
    if constexpr (G::SG == 1) group_dma<G>(smem, P, s + 2, wave, lane);
    else if ((s & (G::SG - 1)) == 0) group_dma<G>(smem, P, s / G::SG + 1, wave, lane);
    const uint8_t* st = smem + (s % G::D) * G::STAGE;
    // this lane's scale bytes: byte 2T of the row's stage dword after the
    // shift by 8 * half serves substep T
    const int grp = s / G::SG;
    const uint8_t* gs = smem + G::OFF_G + (grp % G::NB) * G::GBUF + 4 * s - group_start<G>(grp, P.kblocks);
    int sc[G::TI + G::TJ];
#pragma unroll
    for (int i = 0; i < G::TI; i++)
        sc[i] = (int)(*reinterpret_cast<const uint32_t*>(gs + (ra + 32 * i) * G::GROW) >> (8 * half));
#pragma unroll
    for (int j = 0; j < G::TJ; j++)
        sc[G::TI + j] = (int)(*reinterpret_cast<const uint32_t*>(gs + (G::BM + rb + 32 * j) * G::GROW) >> (8 * half));
    if constexpr (G::MBS == 0) {
        substep<0, G>(acc, st, ra, rb, half, sc);
        substep<1, G>(acc, st, ra, rb, half, sc);
    } else {
        float fb[G::TJ];
#pragma unroll
        for (int j = 0; j < G::TJ; j++) {
            fb[j] = ue4m3(cur[G::TI + j]);
#if defined(__HIP_DEVICE_COMPILE__)
            // without B macro scales fb is 1: kept opaque, so that the fold
            // has the same shape (and register use) as with them
            if constexpr ((G::MBS & 2) == 0) asm volatile("" : "+v"(fb[j]));
#endif
        }
        mbs_stage<G>(acc, st, ra, rb, half, sc, fb);
    }
}

template <bool CBF16, class G>
__global__ __launch_bounds__(64 * G::NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_lds(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, void* __restrict__ C, int64_t M, int64_t N, int64_t K, int64_t ldc,
    const uint8_t* __restrict__ MA, const uint8_t* __restrict__ MB) {
    constexpr int FA = G::FA, FB = G::FB, TI = G::TI, TJ = G::TJ, D = G::D;
    static_assert(2 * G::PW + G::GPW + G::NS <= 63, "vmcnt");
    static_assert(G::SMEM <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[G::SMEM];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, lrow = lane & 31;
    const int wm = wave / G::WGN, wn = wave % G::WGN;

    // tile order: slots dealt to the 8 XCDs round robin, so consecutive tiles
    // of a grouped order land on one XCD and share A and B panels in its L2
    const int tm = (int)((M + G::BM - 1) / G::BM), tn = (int)((N + G::BN - 1) / G::BN);
    const int T = tm * tn;
    int bid = blockIdx.x;
    if (T % 8 == 0) bid = (bid % 8) * (T / 8) + bid / 8;
    constexpr int GM = 8;
    const int group = bid / (GM * tn), first = group * GM;
    const int gsz = (tm - first) < GM ? (tm - first) : GM;
    const int in_g = bid - group * GM * tn;
    const int64_t m0 = (int64_t)(first + in_g % gsz) * G::BM, n0 = (int64_t)(in_g / gsz) * G::BN;

    const int nst = (int)(K / G::BK);
    const int kblocks = (int)(K / 32);
    const int64_t rowa = (int64_t)kblocks * lbb(FA), rowb = (int64_t)kblocks * lbb(FB);
    const int64_t va = M - m0 < G::BM ? M - m0 : G::BM, vb = N - n0 < G::BN ? N - n0 : G::BN;
    const rsrc_t pa = rsrc(A + m0 * rowa, va * rowa), pb = rsrc(B + n0 * rowb, vb * rowb);
    const rsrc_t psa = rsrc(SA + m0 * kblocks, va * kblocks), psb = rsrc(SB + n0 * kblocks, vb * kblocks);
    const rsrc_t z = rsrc(A, 0);
    const int mcols = (int)(K / 128);
    const rsrc_t pma = (G::MBS & 1) ? rsrc(MA + m0 * mcols, va * mcols) : z;
    const rsrc_t pmb = (G::MBS & 2) ? rsrc(MB + n0 * mcols, vb * mcols) : z;

    const int ra = wm * 32 * TI + lrow, rb = wn * 32 * TJ + lrow;   // this lane's operand rows in the tile
    const LPanels P = {pa, pb, psa, psb, z, pma, pmb, rowa, rowb, kblocks, nst, mcols};
    v16f acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    uint32_t mc[G::NS], mn[G::NS];
#pragma unroll
    for (int i = 0; i < G::NS; i++) mc[i] = mn[i] = 0x38u;
    stage_dma<G>(smem, P, 0, wave, lane);
    group_dma<G>(smem, P, 0, wave, lane);
    stage_macro<G>(mc, P, 0, ra, rb);
    stage_dma<G>(smem, P, 1, wave, lane);
    if constexpr (G::SG == 1) group_dma<G>(smem, P, 1, wave, lane);
    for (int s = 0; s < nst; s++) {
        lds_step<G>(smem, P, s, wave, lane, half, ra, rb, acc, mc, mn);
#pragma unroll
        for (int i = 0; i < G::NS; i++) mc[i] = mn[i];
    }
    wait_vm<0>();

    if constexpr (CBF16) {
        // bf16 C through a private 16-row strip of each wave in the ring (free
        // once every wave has read the last stage), then 16-byte row stores
        static_assert(G::NW * CStore<G>::AREA <= G::D * G::STAGE, "C strips fit in the ring");
        __syncthreads();
        store_c_bf16<G, false>(acc, smem + wave * CStore<G>::AREA, C, m0, n0, M, N, ldc, wm, wn, lane, half, lrow);
    } else {
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < TJ; j++) {
                const int64_t n = n0 + wn * 32 * TJ + 32 * j + lrow;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t m = m0 + wm * 32 * TI + 32 * i + 8 * (r / 4) + 4 * half + (r % 4);
                    if (m < M) static_cast<float*>(C)[m * ldc + n] = acc[i][j][r];
                }
            }
    }
}

#ifndef LDS_WGM
#define LDS_WGM 2
#define LDS_WGN 4
#define LDS_TI 4
#define LDS_TJ 2
#endif

template <class G>
hipError_t launch_lds_g(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c, int64_t M,
                        int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s, const uint8_t* ma,
                        const uint8_t* mb) {
    const int64_t tiles = ((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN);
    if (c_bf16) k_gemm_lds<true, G><<<(unsigned)tiles, 64 * G::NW, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc, ma, mb);
    else k_gemm_lds<false, G><<<(unsigned)tiles, 64 * G::NW, 0, s>>>(a, sa, b, sb, c, M, N, K, ldc, ma, mb);
    return hipGetLastError();
}

// the tile of an operand pair: 256 x 256 (8 waves of 4 x 2 MFMA tiles) while
// three stages of both operands fit in LDS; with an 8-bit operand beside a
// 6- or 8-bit one, 128 x 256 (8-bit A) or 256 x 128 (8 waves of 2 x 2 tiles)
template <int FA, int FB, int SG>
struct LPick {
    static constexpr bool big = lbb(FA) + lbb(FB) <= 48;
    static constexpr bool tall = !big && !is_fp8(FA);       // FP6 A, FP8 B: 256 x 128
    using G = LGeo<FA, FB, big ? LDS_WGM : (tall ? 4 : 2), big ? LDS_WGN : (tall ? 2 : 4), big ? LDS_TI : 2,
                   big ? LDS_TJ : 2, 0, SG>;
};

// scale groups of 4 stages need K >= 512 (a whole group fits a scale row)
template <int FA, int FB>
hipError_t launch_lds_t(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c, int64_t M,
                        int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    if (K >= 512)
        return launch_lds_g<typename LPick<FA, FB, 4>::G>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s, nullptr, nullptr);
    return launch_lds_g<typename LPick<FA, FB, 1>::G>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s, nullptr, nullptr);
}

// MXFP4 with macro-block scales on A (MBS 1), B (2) or both (3): the same
// 256 x 256 tiles, with the stage folded tile by tile (mbs_stage)
template <int MBS>
hipError_t launch_lds_mbs_t(const uint8_t* a, const uint8_t* sa, const uint8_t* ma, const uint8_t* b,
                            const uint8_t* sb, const uint8_t* mb, void* c, int64_t M, int64_t N, int64_t K,
                            int64_t ldc, int c_bf16, hipStream_t s) {
    if (K >= 512)
        return launch_lds_g<LGeo<MF_E2M1, MF_E2M1, 2, 4, 4, 2, MBS, 4>>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s, ma, mb);
    return launch_lds_g<LGeo<MF_E2M1, MF_E2M1, 2, 4, 4, 2, MBS, 1>>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s, ma, mb);
}

template <int FA>
hipError_t launch_lds_b(int eb, const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, void* c,
                        int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    switch (lmf(eb)) {
    case 4: return launch_lds_t<FA, 4>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    case 2: return launch_lds_t<FA, 2>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    case 3: return launch_lds_t<FA, 3>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    case 0: return launch_lds_t<FA, 0>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    default: return launch_lds_t<FA, 1>(a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    }
}

}  // namespace

hipError_t launch_gemm_lds(int ea, const uint8_t* a, const uint8_t* sa, int eb, const uint8_t* b, const uint8_t* sb,
                           void* c, int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s,
                           const uint8_t* ma, const uint8_t* mb) {
    if (M == 0 || N == 0) return hipSuccess;
    if (K % 128) return hipErrorInvalidValue;
    if (ma || mb) {
        if (ea != E2M1 || eb != E2M1) return hipErrorInvalidValue;
        if (ma && mb) return launch_lds_mbs_t<3>(a, sa, ma, b, sb, mb, c, M, N, K, ldc, c_bf16, s);
        if (ma) return launch_lds_mbs_t<1>(a, sa, ma, b, sb, mb, c, M, N, K, ldc, c_bf16, s);
        return launch_lds_mbs_t<2>(a, sa, ma, b, sb, mb, c, M, N, K, ldc, c_bf16, s);
    }
    switch (lmf(ea)) {
    case 4: return launch_lds_b<4>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    case 2: return launch_lds_b<2>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    case 3: return launch_lds_b<3>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    case 0: return launch_lds_b<0>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    default: return launch_lds_b<1>(eb, a, sa, b, sb, c, M, N, K, ldc, c_bf16, s);
    }
}

}  // namespace mxk
