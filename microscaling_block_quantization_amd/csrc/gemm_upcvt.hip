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
// codes, multiplies by the block scale -- exactly, since the product has at
// most six significant bits -- and the products run on the fp16 or bf16
// matrix instruction.  (The scaled converts use only the exponent of their
// scale operand, so they apply E8M0 scales directly but not UE4M3 / UE5M3
// ones: measured on gfx950.)  The per-tensor scales multiply the fp32 result
// once at the end.
//
// Two kernels: an LDS-staged one (1 x 16 and 1 x 32 blocks, K a multiple of
// 128; below) and a register-only one for the rest.
//
// Layout of the register-only kernel: a lane of the bf16 instruction supplies
// 8 K-values of its row.  The K order inside one instruction is free as long
// as A and B agree, so lane (row r, half h) takes K = k0 + 32 h + 8 j + (0..7)
// in the j-th of the four instructions of a 64-wide K step: the 16 code bytes
// of k0 + 32 h .. + 31, one load, and every group of 8 lies inside one block
// (blocks are multiples of 8 wide).
#include <type_traits>

#include "mx_kernels.hpp"
#include "gemm_cstore.hpp"

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
    const uint8_t* macro;     // nullable: UE4M3 macro-block scales, rows x K/128 bytes (E8M0 block scales only)
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
    // macro-block scaling: the block's scale times the UE4M3 scale of its 1 x 128
    // macro block (exact in fp32), and the fp32 decode
    const float sm = U.macro ? uscale(U.macro[row * (K / 128) + kb / 128], UK_UE4M3) : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float sc = uscale(srow[(kb + 8 * j) / U.bc], U.kind);
        o[j] = U.macro ? decode8(ww[j], sc * sm) : U.kind == UK_E8M0 ? decode8_pow2(ww[j], sc) : decode8(ww[j], sc);
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

// ---------------------------------------------------------------------------
// LDS-staged form for 1 x 16 and 1 x 32 blocks with K a multiple of 128: 256 x
// 256 tiles of 8 waves (4 x 2 MFMA tiles each), 128-wide K stages of codes (64
// bytes per row, four 16-byte chunks XOR-permuted per row so the chunk reads
// of 16 consecutive rows hit distinct banks) in a three-deep LDS ring filled
// by LDS-DMA two stages ahead, together with the stage's block scales (8
// bytes per row at most), so no load in the loop writes registers.  Each
// lane decodes its 32-code chunk group by group, without branches, and feeds
// the instruction right away.
//
// Two routes.  When both operands carry UE4M3 scales (NVFP4, with or without
// its tensor scale) every product q * s has at most six significant bits and
// lies in [2^-10, 2688]: exact in fp16, so the codes are decoded to fp16 (the
// convert scaled by 2^8, times the scale code shifted into an fp16 bit pattern,
// which is s * 2^-8) and multiplied by the fp16 instruction at the bf16 rate,
// 8 vector operations per 8 codes.  Otherwise (E8M0 or UE5M3 scales on either
// side: products span more binades than fp16 holds) they go to bf16: E8M0 by
// the power-of-two scaled convert, 4 operations per 8 codes; UE4M3 / UE5M3 by
// an fp32 decode times s, narrowed exactly, 16 operations.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

constexpr int UWGM = 2, UWGN = 4, UTI = 4, UTJ = 2, UNW = UWGM * UWGN;
constexpr int UBM = UWGM * 32 * UTI, UBN = UWGN * 32 * UTJ, UD = 3;
constexpr int USA = UBM * 64, UCODES = (UBM + UBN) * 64;   // A codes, then B codes
constexpr int USTAGE = UCODES + (UBM + UBN) * 8;           // then 8 scale bytes per row
constexpr int UPW = UCODES / 1024 / UNW;               // code DMA pieces per wave per stage
constexpr int USW = (UBM + UBN) * 2 / 64 / UNW;        // scale DMA pieces (a dword per lane) per wave

// operand decode kinds of the LDS kernel: E8M0 by the scaled convert; fp8
// scales, or E8M0 times a UE4M3 macro scale, by the fp32 decode; UE4M3 on both
// sides by the fp16 route
enum { DK_E8M0 = 0, DK_FP8 = 1, DK_F16 = 2, DK_MBS = 3 };

__device__ __forceinline__ int uphys(int r, int p) { return p ^ (((r >> 1) & 3) ^ ((r >> 3) & 1)); }

__device__ __forceinline__ rsrc_t ursrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// per-operand constants of the decode
struct UDec {
    float mul;          // DK_FP8: 2^(127 - bias)
    uint32_t nan;       // DK_FP8 / DK_F16: the scale code that means NaN
    int lg;             // log2 of the block width (4 or 5)
};

struct UPanels {
    rsrc_t a, b, sa, sb, z;
    rsrc_t ma, mb;                                      // macro scale panels (DK_MBS operands)
    int rowb, srowa, srowb, spa, spb, nst;              // code row bytes; scale row and stage bytes of A, B
    int mrow;                                           // macro bytes per row (K / 128)
};

template <int N>
__device__ __forceinline__ void uwait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void ubarrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// DMA of stage s (device pass only: the host pass rejects the LDS-DMA builtin
// in a template and would drop the launch stubs): the codes in 16-byte pieces,
// then each row's stage scales, 8 bytes (1 x 32 blocks: 4, twice) a dword per
// lane.  A wave's pieces
// all fall in one operand's panel, so the panel is a select, not a branch, and
// every wave issues the same UPW + USW loads per stage, oldest first, which the
// stage waits count on.
static_assert((USA / 1024) % UPW == 0 && (UBM * 2 / 64) % USW == 0,
              "a wave's DMA pieces must not straddle the two panels");
__device__ __forceinline__ void ustage_dma(uint8_t* smem, const UPanels& P, int s, int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    const rsrc_t pa = P.a, pb = P.b, psa = P.sa, psb = P.sb, pz = P.z;
    const bool in = s < P.nst;
    uint8_t* slot = smem + (s % UD) * USTAGE;
    {
        const bool isb = wave * UPW >= USA / 1024;           // uniform
        const rsrc_t r = in ? (isb ? pb : pa) : pz;
        const int h0 = isb ? wave * UPW - USA / 1024 : wave * UPW;
        uint8_t* base = slot + (isb ? USA : 0);
#pragma unroll
        for (int k = 0; k < UPW; k++) {
            const int f = (h0 + k) * 64 + lane, row = f >> 2, q = f & 3;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(base + (h0 + k) * 1024), 16,
                                                     row * P.rowb + uphys(row, q) * 16, s * 64, 0, 0);
        }
    }
    {
        const bool isb = wave * USW >= UBM * 2 / 64;          // uniform
        const rsrc_t r = in ? (isb ? psb : psa) : pz;
        const int h0 = isb ? wave * USW - UBM * 2 / 64 : wave * USW;
        const int srow = isb ? P.srowb : P.srowa, sp = isb ? P.spb : P.spa;
        uint8_t* base = slot + UCODES + (isb ? UBM * 8 : 0);
#pragma unroll
        for (int k = 0; k < USW; k++) {
            // 1 x 32 blocks: the second dword repeats the first, so that no
            // load reaches past the row's last stage
            const int f = (h0 + k) * 64 + lane, row = f >> 1, d = sp == 8 ? f & 1 : 0;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(base + (h0 + k) * 256), 4, row * srow + 4 * d,
                                                     sp * s, 0, 0);
        }
    }
#endif
}

// eight fp16 products q * s of the codes in dword w; h holds s * 2^-8 twice
template <int BYTE>
__device__ __forceinline__ h2v dec2_f16(uint32_t w, h2v h) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, BYTE) * h;
}
__device__ __forceinline__ h8v dec8_f16(uint32_t w, h2v h) {
    const h2v p0 = dec2_f16<0>(w, h), p1 = dec2_f16<1>(w, h), p2 = dec2_f16<2>(w, h), p3 = dec2_f16<3>(w, h);
    h8v v;
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    return v;
}

// scale operand of one group for each kind: E8M0 an fp32 power of two (code
// 0: 2^-127; 255: NaN); FP8 the fp32 value (subnormal codes through an fp32
// subnormal times 2^(127 - bias), exact); F16 the UE4M3 code's fp16 pattern
// (s * 2^-8, the exponent bias difference) in both halves
template <int DK>
__device__ __forceinline__ uint32_t uscale_bits(uint32_t c, const UDec& d) {
    if constexpr (DK == DK_E8M0 || DK == DK_MBS) {
        const uint32_t v = c ? c << 23 : 0x00400000u;
        return c == 255u ? 0x7fc00000u : v;
    } else if constexpr (DK == DK_FP8) {
        const float v = __uint_as_float(c << 20) * d.mul;
        return c == d.nan ? 0x7fc00000u : __float_as_uint(v);
    } else {
        const uint32_t v = c == d.nan ? 0x7e00u : c << 7;
        return v | (v << 16);
    }
}

template <int DK>
struct UVec {
    typedef typename std::conditional<DK == DK_F16, h8v, bf8v>::type type;
};

// sm: the macro scale of the row's current macro block (DK_MBS; else unused)
template <int DK>
__device__ __forceinline__ typename UVec<DK>::type udecode(uint32_t w, uint32_t sb, float sm) {
    if constexpr (DK == DK_E8M0) return decode8_pow2(w, __uint_as_float(sb));
    else if constexpr (DK == DK_FP8) return decode8(w, __uint_as_float(sb));
    else if constexpr (DK == DK_MBS) return decode8(w, __uint_as_float(sb) * sm);
    else return dec8_f16(w, __builtin_bit_cast(h2v, sb));
}

// the UE4M3 macro scales of this lane's row tiles for one 128-wide stage: one
// byte per row, read through a resource over the tile's valid rows (rows past
// the end read as 0)
template <int R>
__device__ __forceinline__ void load_macro(float (&m)[R], rsrc_t r, int row0, int mrow, int s) {
#pragma unroll
    for (int i = 0; i < R; i++)
        m[i] = uscale((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (row0 + 32 * i) * mrow + s, 0, 0), UK_UE4M3);
}

// the scale byte of group q (8 codes) of this lane's chunk, from the chunk's
// scale bytes x (1 x 16 blocks: 2 bytes; 1 x 32: 1)
__device__ __forceinline__ uint32_t ugroup_code(uint32_t x, int q, int lg) {
    return (x >> (8 * ((q >> 1) & (lg == 4 ? 1 : 0)))) & 0xffu;
}

// One stage.  With macro scales (DK_MBS), ma / mb hold the stage's macro
// values; the next stage's are loaded after the barrier, before the DMA of
// stage s + 2, so the wait of the next step (for stage s + 1, with the DMA of
// s + 2 in flight) covers them.
template <int KA, int KB>
__device__ __forceinline__ void ustep(uint8_t* smem, const UPanels& P, int s, int wave, int lane, int half, int ra,
                                      int rb, const UDec& da, const UDec& db, v16f (&acc)[UTI][UTJ],
                                      float (&ma)[UTI], float (&mb)[UTJ], float (&na)[UTI], float (&nb)[UTJ]) {
    uwait_vm<UPW + USW>();
    ubarrier();
    if constexpr (KA == DK_MBS) load_macro<UTI>(na, P.ma, ra, P.mrow, s + 1 < P.nst ? s + 1 : s);
    if constexpr (KB == DK_MBS) load_macro<UTJ>(nb, P.mb, rb, P.mrow, s + 1 < P.nst ? s + 1 : s);
    ustage_dma(smem, P, s + 2, wave, lane);
    const uint8_t* st = smem + (s % UD) * USTAGE;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const int c = 2 * t + half;
        // the dword of each row's stage scales that holds chunk c's (1 x 16
        // blocks: bytes 2c, 2c + 1, in dword t; 1 x 32: byte c, in dword 0),
        // shifted to put them at the bottom
        const int oa = da.lg == 4 ? 4 * t : 0, ob = db.lg == 4 ? 4 * t : 0;
        const int sha = da.lg == 4 ? 16 * half : 8 * c, shb = db.lg == 4 ? 16 * half : 8 * c;
        u32x4v xa[UTI], xb[UTJ];
        uint32_t ca[UTI], cb[UTJ];
#pragma unroll
        for (int i = 0; i < UTI; i++) {
            const int r = ra + 32 * i;
            xa[i] = *reinterpret_cast<const u32x4v*>(st + r * 64 + uphys(r, c) * 16);
            ca[i] = *reinterpret_cast<const uint32_t*>(st + UCODES + r * 8 + oa) >> sha;
        }
#pragma unroll
        for (int j = 0; j < UTJ; j++) {
            const int r = rb + 32 * j;
            xb[j] = *reinterpret_cast<const u32x4v*>(st + USA + r * 64 + uphys(r, c) * 16);
            cb[j] = *reinterpret_cast<const uint32_t*>(st + UCODES + (UBM + r) * 8 + ob) >> shb;
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            typename UVec<KA>::type a[UTI];
            typename UVec<KB>::type b[UTJ];
#pragma unroll
            for (int i = 0; i < UTI; i++)
                a[i] = udecode<KA>(xa[i][q], uscale_bits<KA>(ugroup_code(ca[i], q, da.lg), da), ma[i]);
#pragma unroll
            for (int j = 0; j < UTJ; j++)
                b[j] = udecode<KB>(xb[j][q], uscale_bits<KB>(ugroup_code(cb[j], q, db.lg), db), mb[j]);
#pragma unroll
            for (int i = 0; i < UTI; i++)
#pragma unroll
                for (int j = 0; j < UTJ; j++) {
                    if constexpr (KA == DK_F16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                }
        }
    }
}

// the wave tiles of k_gemm_upcvt_lds as the shared C store path sees them
struct UCGeo {
    static constexpr int TI = UTI, TJ = UTJ, BM = UBM;
};

template <bool CBF16, int KA, int KB>
__global__ __launch_bounds__(64 * UNW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_upcvt_lds(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, UDec da, UDec db, const float* ta, const float* tb, void* __restrict__ C,
    int64_t M, int64_t N, int64_t K, int64_t ldc, const uint8_t* __restrict__ MA, const uint8_t* __restrict__ MB) {
    static_assert((KA == DK_F16) == (KB == DK_F16), "the fp16 route needs both operands in fp16");
    __shared__ __attribute__((aligned(16))) uint8_t smem[UD * USTAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, lrow = lane & 31;
    const int wm = wave / UWGN, wn = wave % UWGN;
    // XCD-aware grouped tile order
    const int tm = (int)((M + UBM - 1) / UBM), tn = (int)((N + UBN - 1) / UBN);
    const int T = tm * tn;
    int bid = blockIdx.x;
    if (T % 8 == 0) bid = (bid % 8) * (T / 8) + bid / 8;
    constexpr int GM = 8;
    const int group = bid / (GM * tn), first = group * GM;
    const int gsz = (tm - first) < GM ? (tm - first) : GM;
    const int in_g = bid - group * GM * tn;
    const int64_t m0 = (int64_t)(first + in_g % gsz) * UBM, n0 = (int64_t)(in_g / gsz) * UBN;

    const int rowb = (int)(K / 2), srowa = (int)(K >> da.lg), srowb = (int)(K >> db.lg);
    const int64_t va = M - m0 < UBM ? M - m0 : UBM, vb = N - n0 < UBN ? N - n0 : UBN;
    UPanels P;
    P.a = ursrc(A + m0 * rowb, va * rowb);
    P.b = ursrc(B + n0 * rowb, vb * rowb);
    P.sa = ursrc(SA + m0 * srowa, va * srowa);
    P.sb = ursrc(SB + n0 * srowb, vb * srowb);
    P.z = ursrc(A, 0);
    P.rowb = rowb;
    P.srowa = srowa;
    P.srowb = srowb;
    P.spa = 128 >> da.lg;
    P.spb = 128 >> db.lg;
    P.nst = (int)(K / 128);
    P.mrow = (int)(K / 128);
    P.ma = KA == DK_MBS ? ursrc(MA + m0 * P.mrow, va * P.mrow) : P.z;
    P.mb = KB == DK_MBS ? ursrc(MB + n0 * P.mrow, vb * P.mrow) : P.z;

    const int ra = wm * 32 * UTI + lrow, rb = wn * 32 * UTJ + lrow;
    v16f acc[UTI][UTJ];
#pragma unroll
    for (int i = 0; i < UTI; i++)
#pragma unroll
        for (int j = 0; j < UTJ; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    // macro scales of stage 0 go out before its DMA, so its wait covers them
    float ma[UTI], mb[UTJ], na[UTI], nb[UTJ];
#pragma unroll
    for (int i = 0; i < UTI; i++) ma[i] = na[i] = 1.0f;
#pragma unroll
    for (int j = 0; j < UTJ; j++) mb[j] = nb[j] = 1.0f;
    if constexpr (KA == DK_MBS) load_macro<UTI>(ma, P.ma, ra, P.mrow, 0);
    if constexpr (KB == DK_MBS) load_macro<UTJ>(mb, P.mb, rb, P.mrow, 0);
    ustage_dma(smem, P, 0, wave, lane);
    ustage_dma(smem, P, 1, wave, lane);
    for (int s = 0; s < P.nst; s++) {
        ustep<KA, KB>(smem, P, s, wave, lane, half, ra, rb, da, db, acc, ma, mb, na, nb);
#pragma unroll
        for (int i = 0; i < UTI; i++) ma[i] = na[i];
#pragma unroll
        for (int j = 0; j < UTJ; j++) mb[j] = nb[j];
    }
    uwait_vm<0>();

    const float g = (ta ? *ta : 1.0f) * (tb ? *tb : 1.0f);
#pragma unroll
    for (int i = 0; i < UTI; i++)
#pragma unroll
        for (int j = 0; j < UTJ; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = acc[i][j][r] * g;
    if constexpr (CBF16) {
        // bf16 C through a private 16-row strip of each wave in the ring (free
        // once every wave has read the last stage), then 16-byte row stores
        static_assert(UNW * CStore<UCGeo>::AREA <= UD * USTAGE, "C strips fit in the ring");
        __syncthreads();
        store_c_bf16<UCGeo, false>(acc, smem + wave * CStore<UCGeo>::AREA, C, m0, n0, M, N, ldc, wm, wn, lane, half, lrow);
    } else {
#pragma unroll
        for (int i = 0; i < UTI; i++)
#pragma unroll
            for (int j = 0; j < UTJ; j++) {
                const int64_t n = n0 + wn * 32 * UTJ + 32 * j + lrow;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t m = m0 + wm * 32 * UTI + 32 * i + 8 * (r / 4) + 4 * half + (r % 4);
                    if (m < M) static_cast<float*>(C)[m * ldc + n] = acc[i][j][r];
                }
            }
    }
}

UDec udec(const UOperand& U) {
    UDec d;
    d.mul = U.kind == UK_UE5M3 ? 0x1p112f : 0x1p120f;
    d.nan = U.kind == UK_UE5M3 ? 0xffu : 0x7fu;
    d.lg = U.bc == 16 ? 4 : 5;
    return d;
}

template <int KA, int KB>
hipError_t launch_upcvt_lds_t(const UOperand& A, const UOperand& B, const float* ta, const float* tb, void* c,
                              int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    const int64_t tiles = ((M + UBM - 1) / UBM) * ((N + UBN - 1) / UBN);
    const UDec da = udec(A), db = udec(B);
    if (c_bf16)
        k_gemm_upcvt_lds<true, KA, KB><<<(unsigned)tiles, 64 * UNW, 0, s>>>(A.codes, A.scales, B.codes, B.scales, da,
                                                                          db, ta, tb, c, M, N, K, ldc, A.macro, B.macro);
    else
        k_gemm_upcvt_lds<false, KA, KB><<<(unsigned)tiles, 64 * UNW, 0, s>>>(A.codes, A.scales, B.codes, B.scales, da,
                                                                           db, ta, tb, c, M, N, K, ldc, A.macro,
                                                                           B.macro);
    return hipGetLastError();
}

hipError_t launch_upcvt_lds(const UOperand& A, const UOperand& B, const float* ta, const float* tb, void* c,
                            int64_t M, int64_t N, int64_t K, int64_t ldc, int c_bf16, hipStream_t s) {
    // macro-block scaled operands (E8M0 block scales) against E8M0 ones
    if (A.macro || B.macro) {
        if (A.kind != UK_E8M0 || B.kind != UK_E8M0) return hipErrorInvalidValue;
        if (A.macro && B.macro) return launch_upcvt_lds_t<DK_MBS, DK_MBS>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
        if (A.macro) return launch_upcvt_lds_t<DK_MBS, DK_E8M0>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
        return launch_upcvt_lds_t<DK_E8M0, DK_MBS>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
    }
    if (A.kind == UK_UE4M3 && B.kind == UK_UE4M3)
        return launch_upcvt_lds_t<DK_F16, DK_F16>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
    const bool pa = A.kind == UK_E8M0, pb = B.kind == UK_E8M0;
    if (pa && pb) return launch_upcvt_lds_t<DK_E8M0, DK_E8M0>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
    if (pa) return launch_upcvt_lds_t<DK_E8M0, DK_FP8>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
    if (pb) return launch_upcvt_lds_t<DK_FP8, DK_E8M0>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
    return launch_upcvt_lds_t<DK_FP8, DK_FP8>(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
}

}  // namespace

bool gemm_upcvt_scale_ok(int scale) {
    return scale == SC_E8M0 || scale == SC_UE4M3 || scale == SC_NVFP4 || scale == SC_UE5M3;
}

hipError_t launch_gemm_upcvt(int sca, int bca, const uint8_t* a, const uint8_t* sa, const float* ta, int scb, int bcb,
                             const uint8_t* b, const uint8_t* sb, const float* tb, void* c, int64_t M, int64_t N,
                             int64_t K, int64_t ldc, int c_bf16, hipStream_t s, const uint8_t* ma,
                             const uint8_t* mb) {
    if (M == 0 || N == 0) return hipSuccess;
    if (!gemm_upcvt_scale_ok(sca) || !gemm_upcvt_scale_ok(scb) || bca % 8 || bcb % 8 || K % 32)
        return hipErrorInvalidValue;
    if ((ma || mb) && (K % 128 || sca != SC_E8M0 || scb != SC_E8M0)) return hipErrorInvalidValue;
    const UOperand A = {a, sa, ukind(sca), bca, ma};
    const UOperand B = {b, sb, ukind(scb), bcb, mb};
    if (K % 128 == 0 && (bca == 16 || bca == 32) && (bcb == 16 || bcb == 32))
        return launch_upcvt_lds(A, B, ta, tb, c, M, N, K, ldc, c_bf16, s);
    dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
    if (c_bf16) k_gemm_upcvt<true><<<grid, 256, 0, s>>>(A, B, ta, tb, c, M, N, K, ldc);
    else k_gemm_upcvt<false><<<grid, 256, 0, s>>>(A, B, ta, tb, c, M, N, K, ldc);
    return hipGetLastError();
}

}  // namespace mxk
