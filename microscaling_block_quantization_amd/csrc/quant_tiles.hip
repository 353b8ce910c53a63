// quant_tiles.hip -- quantization of b x 1 (column) and b x b (2D) blocks on
// gfx950, b in {8, 16, 32} (the block organisations of the ARITH 2025
// MX-training report, main results 5: column blocks for activations, 2D blocks
// as the balance).
//
// A workgroup owns a band of b rows and 1 KiB of each of them (512 bf16 or 256
// fp32 columns) and stages it in LDS with coalesced 16-byte loads: every load
// of a wave is one 1 KiB row segment.  Then
//  pass 1  each thread reduces its columns (two bf16 columns, or one fp32
//          column: one LDS word per row) down the b rows; the lanes of a 2D
//          block combine their maxima by shuffles.  The block's scale goes to
//          memory and, packed with the kind of scaling and the offset, into an
//          LDS parameter word per column;
//  pass 2  each thread re-reads 16-byte row chunks of the band from LDS,
//          rounds them with their columns' parameters and writes codes and
//          dequantized values row-major, so every store of a wave is
//          coalesced as well.
// Codes keep the row-block layout (element (r, c) where a row block puts it);
// the scale grid is (rows / b) x (cols / bc).  Statistics accumulate per
// chunk in fp32 (float64 when a chunk's sums leave the fp32 range) and per
// thread in float64; a block counts as all-zero when every dequantized value
// of it is zero, which the chunks record in an LDS bit mask per column.
#include "mx_kernels.hpp"

namespace mxk {
using namespace mxd;

namespace {

constexpr int TROW = 1024;                     // bytes of one band row in LDS
typedef float f2vr __attribute__((ext_vector_type(2)));

// kinds of block scaling, in the LDS parameter word of a column
enum { K_POW2 = 0, K_DIV = 1, K_ZERO = 2, K_NAN = 3 };

__device__ __forceinline__ uint32_t pack_prm(int code, int kind, uint16_t off) {
    return (uint32_t)(code & 0xff) | ((uint32_t)kind << 8) | ((uint32_t)off << 16);
}

template <bool BF>
__device__ __forceinline__ float word_elem(uint32_t w, int j) {
    if constexpr (BF) return j ? bf16hi(w) : bf16lo(w);
    else return __uint_as_float(w);
}

// TM fixes the element kind, and with it the pass-2 route, at compile time:
// 0 any format; 1 E2M1 with E8M0 or E3M0 scales, to nearest or stochastic
// (the pair convert or the bit-level SR decision); 2 INT4 with E8M0 scales to
// nearest.  The code of the other kinds and widths then drops out of the loop.
template <bool BF, int BR, int TM>
__global__ __launch_bounds__(NT) void k_tiles(QParams p) {
    constexpr int CPT = BF ? 2 : 1;            // columns per thread in pass 1
    constexpr int TC = TROW / (BF ? 2 : 4);    // columns of the tile
    constexpr int EPC = BF ? 8 : 4;            // elements per 16-byte chunk
    constexpr int NCH = BR * (TROW / 16);      // chunks of the band
    __shared__ __attribute__((aligned(16))) uint8_t tile[BR * TROW];
    __shared__ __attribute__((aligned(16))) uint32_t prm[TC];
    __shared__ uint32_t zmask[TC / 32];

    const Elem E = make_elem(TM == 1 ? E2M1 : (TM == 2 ? INT4 : p.elem), p.asym);
    const int scale = TM == 2 ? SC_E8M0 : p.scale;
    const int round = TM == 2 ? RTNE : p.round;
    const int tid = threadIdx.x;
    const int64_t ctiles = (p.cols + TC - 1) / TC;
    const int64_t band = blockIdx.x / ctiles;
    const int64_t col0 = (blockIdx.x - band * ctiles) * TC;
    const int64_t r0 = band * BR;
    const int ncol = (int)(p.cols - col0 < TC ? p.cols - col0 : TC);   // a multiple of 8 and of bc
    const char* xin = static_cast<const char*>(p.x);

    // ---- stage the band: chunk k is row k / 64, 16-byte piece k % 64 -------
#pragma unroll
    for (int k = tid; k < NCH; k += NT) {
        const int row = k >> 6, pc = k & 63;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (pc * EPC < ncol) w = ld_stream16(xin + ((r0 + row) * p.ld + col0 + pc * EPC) * (BF ? 2 : 4));
        *reinterpret_cast<u32x4*>(tile + row * TROW + pc * 16) = w;
    }
    if (tid < TC / 32) zmask[tid] = ~0u;
    __syncthreads();

    const bool two_d = p.bc > 1;
    constexpr int G1 = BR / CPT;               // lanes of one 2D block in pass 1
    const float g = (scale == SC_NVFP4) ? *p.tensor_scale : 1.0f;
    const int eref = (scale == SC_E3M0) ? *p.ref_exp : 0;
    const bool ue5 = scale == SC_UE5M3;

    // ---- pass 1: block maxima and scales -------------------------------------
    {
        float amax[CPT], mn[CPT], mx[CPT];
        int fin[CPT];
#pragma unroll
        for (int j = 0; j < CPT; j++) { amax[j] = 0.f; mn[j] = INFINITY; mx[j] = -INFINITY; fin[j] = 1; }
#pragma unroll
        for (int row = 0; row < BR; row++) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(tile + row * TROW)[tid];
#pragma unroll
            for (int j = 0; j < CPT; j++) {
                const float v = word_elem<BF>(w, j);
                if (!finitef(v)) { fin[j] = 0; continue; }
                amax[j] = fmaxf(amax[j], fabsf(v));
                mn[j] = fminf(mn[j], v);
                mx[j] = fmaxf(mx[j], v);
            }
        }
        if (two_d) {
            float a = amax[0], lo = mn[0], hi = mx[0];
            int f = fin[0];
#pragma unroll
            for (int j = 1; j < CPT; j++) { a = fmaxf(a, amax[j]); lo = fminf(lo, mn[j]); hi = fmaxf(hi, mx[j]); f &= fin[j]; }
            a = group_max<G1>(a);
            f = group_and<G1>(f);
            lo = group_min<G1>(lo);
            hi = group_max<G1>(hi);
#pragma unroll
            for (int j = 0; j < CPT; j++) { amax[j] = a; mn[j] = lo; mx[j] = hi; fin[j] = f; }
        }
        int kind[CPT], e[CPT], sc[CPT];
        uint16_t ob[CPT];
        float o[CPT];
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            kind[j] = K_POW2; e[j] = 0; sc[j] = 0; ob[j] = 0; o[j] = 0.f;
            if (!fin[j]) {
                kind[j] = K_NAN;
                sc[j] = (scale == SC_UE4M3 || scale == SC_NVFP4) ? 0x7f : 0xff;
            } else if (p.asym) {
                if (E.kind == INT4) {
                    ob[j] = bf16_floor(mn[j]);
                    o[j] = bf16f(ob[j]);
                    const float R = mx[j] - o[j];
                    e[j] = R > 0.f ? e8m0_exp(p.rule, p.tau, E, R) : -127;
                } else {
                    // the mid-range, each end halved first so that it cannot overflow
                    ob[j] = bf16_rne(mx[j] * 0.5f + mn[j] * 0.5f);
                    o[j] = bf16f(ob[j]);
                }
            } else if (scale == SC_E8M0) {
                e[j] = e8m0_exp(p.rule, p.tau, E, amax[j]);
            } else if (scale == SC_E3M0) {
                int cdown = 7;
                if (amax[j] > 0.f) {
                    cdown = eref - e_ceil(amax[j], E.qmax);
                    cdown = cdown < 0 ? 0 : (cdown > 7 ? 7 : cdown);
                }
                e[j] = eref - cdown;
                sc[j] = cdown;
            } else {
                float t = amax[j] / E.qmax;
                if (scale == SC_NVFP4) t = t / g;
                sc[j] = fp8_code(ue5, t);
                const float sbv = fp8_value(ue5, sc[j]);
                kind[j] = ((scale == SC_NVFP4 ? sbv * g : sbv) == 0.f) ? K_ZERO : K_DIV;
            }
        }
        if (p.asym && E.kind != INT4) {
            // E2M1 with an offset: the exponent comes from max |x - o| over the block
            float ym[CPT];
#pragma unroll
            for (int j = 0; j < CPT; j++) ym[j] = 0.f;
#pragma unroll
            for (int row = 0; row < BR; row++) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(tile + row * TROW)[tid];
#pragma unroll
                for (int j = 0; j < CPT; j++) ym[j] = fmaxf(ym[j], fabsf(word_elem<BF>(w, j) - o[j]));
            }
            if (two_d) {
                float a = ym[0];
#pragma unroll
                for (int j = 1; j < CPT; j++) a = fmaxf(a, ym[j]);
                a = group_max<G1>(a);
#pragma unroll
                for (int j = 0; j < CPT; j++) ym[j] = a;
            }
#pragma unroll
            for (int j = 0; j < CPT; j++)
                if (kind[j] == K_POW2) e[j] = e8m0_exp(p.rule, p.tau, E, ym[j]);
        }
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            // the E8M0 code of a power-of-two scale (E3M0 keeps its step-down
            // code; pass 2 rebuilds e from it)
            if (kind[j] == K_POW2 && scale != SC_E3M0) sc[j] = e[j] + 127;
            prm[tid * CPT + j] = pack_prm(sc[j], kind[j], kind[j] == K_NAN ? (uint16_t)0 : ob[j]);
        }
        const int col = tid * CPT;
        if (col < ncol) {
            if (two_d) {
                if (tid % G1 == 0) {
                    const int64_t sidx = band * (p.cols / BR) + (col0 + col) / BR;
                    p.scales[sidx] = (uint8_t)sc[0];
                    if (p.asym) p.offsets[sidx] = kind[0] == K_NAN ? (uint16_t)0 : ob[0];
                }
            } else {
#pragma unroll
                for (int j = 0; j < CPT; j++) {
                    const int64_t sidx = band * p.cols + col0 + col + j;
                    p.scales[sidx] = (uint8_t)sc[j];
                    if (p.asym) p.offsets[sidx] = kind[j] == K_NAN ? (uint16_t)0 : ob[j];
                }
            }
        }
    }
    __syncthreads();

    // ---- pass 2: round, store codes and dequantized values, statistics --------
    double s2 = 0, e2 = 0;
    unsigned long long nz = 0, fl = 0, zb = 0;
    const int64_t crow = code_row_bytes(E.bits, p.cols);
    // Chunk k of the band is row k / 64, piece k % 64, and a thread visits k =
    // tid, tid + NT, ...: always the same piece, so the same EPC columns.
    // Their parameters are unpacked once: down = 2^-e and up = 2^e for a
    // power-of-two scale (the divisor S and s_b for an fp8 one) and the offset.
    const int pc = tid & 63, cl = pc * EPC;       // first column of the piece in the tile
    if (cl < ncol) {
        int kd[EPC], scd[EPC];
        float dn[EPC], upv[EPC], of[EPC];
        bool allpow2 = true;
#pragma unroll
        for (int j = 0; j < EPC; j++) {
            const uint32_t pw = prm[cl + j];
            scd[j] = (int)(pw & 0xff);
            kd[j] = (int)((pw >> 8) & 0xff);
            of[j] = bf16f((uint16_t)(pw >> 16));
            if (kd[j] == K_POW2) {
                const int e = scale == SC_E3M0 ? eref - scd[j] : scd[j] - 127;
                dn[j] = pow2f(-e);
                upv[j] = pow2f(e);
            } else {
                const float sb = fp8_value(ue5, scd[j]);
                dn[j] = scale == SC_NVFP4 ? sb * g : sb;
                upv[j] = sb;
            }
            allpow2 = allpow2 && kd[j] == K_POW2;
        }
        // E2M1 with power-of-two scales: to nearest by the pair convert on the
        // scaled values (round to nearest even, saturating, signed zero kept),
        // stochastically by sr_e2m1; then the pair decode, as the row kernels do
        const bool hwc = E.kind == E2M1 && (round == RTNE || round == SR) && allpow2;
        // INT4 to nearest with power-of-two scales: the integer nearest |v|
        // (ties to even), capped at the largest code; the unsigned variant
        // takes a negative v as zero, the signed one keeps the sign in two's
        // complement (the general encode and decode, written out)
        const bool i4 = E.kind == INT4 && round == RTNE && allpow2;
#pragma unroll 1
        for (int row = tid >> 6; row < BR; row += NT / 64) {
            const int64_t r = r0 + row, c0 = col0 + cl;
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + row * TROW + pc * 16);
            uint32_t rnd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (round == SR) {
                const uint64_t idx = (uint64_t)(r * p.cols + c0);
                draws8(p.seed, p.off, idx >> 3, rnd);
                if (!BF && (idx & 4)) {
                    rnd[0] = rnd[4]; rnd[1] = rnd[5]; rnd[2] = rnd[6]; rnd[3] = rnd[7];
                }
            }
            int code[EPC];
            float d[EPC], xs[EPC];
            uint32_t nzmask = 0;
#pragma unroll
            for (int j = 0; j < EPC; j++) xs[j] = BF ? word_elem<true>(w[j >> 1], j & 1) : __uint_as_float(w[j]);
            if (hwc) {
                float v[EPC];
#pragma unroll
                for (int j = 0; j < EPC; j++) v[j] = (p.asym ? (xs[j] - of[j]) : xs[j]) * dn[j];
                uint32_t cw = 0;
                f2vr dq[EPC / 2];
                if (round == SR) {
#pragma unroll
                    for (int j = 0; j < EPC; j++) cw |= (uint32_t)sr_e2m1(v[j], rnd[j]) << (4 * j);
                } else {
                    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[0], v[1], 1.0f, 0);
                    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[2], v[3], 1.0f, 1);
                    if constexpr (BF) {
                        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[4], v[5], 1.0f, 2);
                        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[6], v[7], 1.0f, 3);
                    }
                }
                dq[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
                dq[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
                if constexpr (BF) {
                    dq[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
                    dq[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
                }
#pragma unroll
                for (int q = 0; q < EPC / 2; q++) {
                    d[2 * q] = dq[q][0] * upv[2 * q];
                    d[2 * q + 1] = dq[q][1] * upv[2 * q + 1];
                }
#pragma unroll
                for (int j = 0; j < EPC; j++) {
                    if (p.asym) d[j] = d[j] + of[j];
                    code[j] = (int)((cw >> (4 * j)) & 0xfu);
                }
            } else if (i4) {
                const float qcap = (float)E.maxidx;
#pragma unroll
                for (int j = 0; j < EPC; j++) {
                    const float v = (p.asym ? (xs[j] - of[j]) : xs[j]) * dn[j];
                    const bool neg = (fbits(v) >> 31) != 0;
                    const float m = (p.asym && neg) ? 0.f : fabsf(v);
                    const int idx = (int)fminf(rintf(m), qcap);
                    const int sv = (!p.asym && neg) ? -idx : idx;
                    code[j] = p.asym ? idx : (sv & 0xf);
                    d[j] = (float)sv * upv[j];
                    if (p.asym) d[j] = d[j] + of[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < EPC; j++) {
                    int c;
                    float dv;
                    if (kd[j] == K_NAN) {
                        c = 0;
                        dv = __uint_as_float(0x7fc00000u);
                    } else if (kd[j] == K_POW2) {
                        const float v = (p.asym ? (xs[j] - of[j]) : xs[j]) * dn[j];
                        c = encode(E, round, v, rnd[j]);
                        dv = decode(E, c) * upv[j];
                        if (p.asym) dv = dv + of[j];
                    } else {
                        const float v = kd[j] == K_ZERO ? ((fbits(xs[j]) >> 31) ? -0.f : 0.f) : xs[j] / dn[j];
                        c = encode(E, kd[j] == K_ZERO ? RTNE : round, v, rnd[j]);
                        dv = decode(E, c) * upv[j];
                        if (scale == SC_NVFP4) dv = dv * g;
                    }
                    code[j] = c;
                    d[j] = dv;
                }
            }
#pragma unroll
            for (int j = 0; j < EPC; j++) nzmask |= (d[j] != 0.f ? 1u : 0u) << j;
            if (nzmask) atomicAnd(&zmask[cl >> 5], ~(nzmask << (cl & 31)));
            if (p.parts) {
                float s2c = 0.f, e2c = 0.f;
#pragma unroll
                for (int j = 0; j < EPC; j++) {
                    const float rj = xs[j] - d[j];
                    s2c = __builtin_fmaf(xs[j], xs[j], s2c);
                    e2c = __builtin_fmaf(rj, rj, e2c);
                    nz += (xs[j] != 0.f);
                    fl += (xs[j] != 0.f && d[j] == 0.f);
                }
                if (fabsf(s2c) < INFINITY && fabsf(e2c) < INFINITY) {
                    s2 += (double)s2c;
                    e2 += (double)e2c;
                } else {
                    // a square beyond the fp32 range (or a NaN): this chunk in float64
#pragma unroll
                    for (int j = 0; j < EPC; j++) {
                        const double xd = xs[j], dd = d[j];
                        s2 += xd * xd;
                        e2 += (xd - dd) * (xd - dd);
                    }
                }
            }
            uint8_t* crw = p.codes + r * crow;
            if (E.bits == 4) {
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < EPC; j++) word |= (uint32_t)(code[j] & 0xf) << (4 * j);
                if constexpr (BF) *reinterpret_cast<uint32_t*>(crw + c0 / 2) = word;
                else *reinterpret_cast<uint16_t*>(crw + c0 / 2) = (uint16_t)word;
            } else if (E.bits == 6) {
                uint64_t bw = 0;
#pragma unroll
                for (int j = 0; j < EPC; j++) bw |= (uint64_t)(code[j] & 0x3f) << (6 * j);
                uint8_t* dst = crw + c0 * 3 / 4;
                if constexpr (BF) {
                    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
                    d16[0] = (uint16_t)bw; d16[1] = (uint16_t)(bw >> 16); d16[2] = (uint16_t)(bw >> 32);
                } else {
                    dst[0] = (uint8_t)bw; dst[1] = (uint8_t)(bw >> 8); dst[2] = (uint8_t)(bw >> 16);
                }
            } else {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int j = 0; j < 4; j++) lo |= (uint32_t)(code[j] & 0xff) << (8 * j);
                if constexpr (BF) {
#pragma unroll
                    for (int j = 0; j < 4; j++) hi |= (uint32_t)(code[4 + j] & 0xff) << (8 * j);
                    *reinterpret_cast<uint2*>(crw + c0) = make_uint2(lo, hi);
                } else {
                    *reinterpret_cast<uint32_t*>(crw + c0) = lo;
                }
            }
            if (p.dq) {
                if (p.dq_bf16) {
                    uint16_t* dst = static_cast<uint16_t*>(p.dq) + r * p.cols + c0;
                    uint32_t pk[EPC / 2];
#pragma unroll
                    for (int j = 0; j < EPC / 2; j++) pk[j] = bf16_rne(d[2 * j]) | ((uint32_t)bf16_rne(d[2 * j + 1]) << 16);
                    if constexpr (BF) *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                    else *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
                } else {
                    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.dq) + r * p.cols + c0);
                    dst[0] = make_float4(d[0], d[1], d[2], d[3]);
                    if constexpr (BF) dst[1] = make_float4(d[4], d[5], d[6], d[7]);
                }
            }
        }
    }
    __syncthreads();

    // ---- all-zero blocks -------------------------------------------------------
    {
        const int col = tid * CPT;
        const uint32_t full = (1u << CPT) - 1u;
        const uint32_t bits = (zmask[col >> 5] >> (col & 31)) & full;
        if (two_d) {
            // the G1 lanes of a block hold its columns: all of their bits set
            const int allz = group_and<G1>(bits == full ? 1 : 0);
            if (col < ncol && tid % G1 == 0) zb += (unsigned long long)allz;
        } else if (col < ncol) {
            zb += (unsigned long long)__builtin_popcount(bits);
        }
    }
    if (p.parts) block_stats<NT>(s2, e2, nz, fl, zb, p.parts + blockIdx.x);
}

constexpr int64_t tile_cols(int in_bf16) { return in_bf16 ? TROW / 2 : TROW / 4; }

}  // namespace

int64_t tiles_grid(const QParams& p) {
    const int64_t tc = tile_cols(p.in_bf16);
    return (p.rows / p.br) * ((p.cols + tc - 1) / tc);
}

hipError_t launch_tiles(const QParams& p, hipStream_t s) {
    const int64_t grid = tiles_grid(p);
    if (grid == 0) return hipSuccess;
    const int tm = (p.elem == E2M1 && (p.round == RTNE || p.round == SR) && (p.scale == SC_E8M0 || p.scale == SC_E3M0))
                       ? 1
                       : ((p.elem == INT4 && p.round == RTNE && p.scale == SC_E8M0) ? 2 : 0);
#define MX_TILE_CASE(BFv, BRv, TMv)                                         \
    if (p.in_bf16 == (BFv) && p.br == (BRv) && tm == (TMv)) {               \
        k_tiles<BFv, BRv, TMv><<<grid, NT, 0, s>>>(p);                      \
        return hipGetLastError();                                           \
    }
#define MX_TILE_TM(BFv, BRv) MX_TILE_CASE(BFv, BRv, 0) MX_TILE_CASE(BFv, BRv, 1) MX_TILE_CASE(BFv, BRv, 2)
    MX_TILE_TM(true, 8) MX_TILE_TM(true, 16) MX_TILE_TM(true, 32)
    MX_TILE_TM(false, 8) MX_TILE_TM(false, 16) MX_TILE_TM(false, 32)
#undef MX_TILE_TM
#undef MX_TILE_CASE
    return hipErrorInvalidValue;
}

}  // namespace mxk
