// quant_tiles.hip -- quantization of b x 1 (column) and b x b (2D) blocks on
// gfx950, b in {8, 16, 32} (the block organisations of the ARITH 2025
// MX-training report, main results 5: column blocks for activations, 2D blocks
// as the balance).
//
// One thread owns V consecutive columns (one 16-byte load per row: 8 bf16 or
// 4 fp32) of one b-row band and keeps the b rows in registers as raw words,
// so the band is read from HBM once and every load of a wave is a coalesced
// 1 KiB row segment.  Column maxima reduce inside the thread; a 2D block
// spans b/V neighbouring lanes that combine their maxima by shuffles.  Codes
// stay row-major (element (r, c) at the same place as for row blocks), so the
// down-column reduction never needs a transposed store.
#include "mx_kernels.hpp"

namespace mxk {
using namespace mxd;

namespace {

template <bool BF>
__device__ __forceinline__ float word_elem(const uint32_t* w, int i) {
    if constexpr (BF) return (i & 1) ? bf16hi(w[i >> 1]) : bf16lo(w[i >> 1]);
    else return __uint_as_float(w[i]);
}

template <bool BF, int BR>
__global__ __launch_bounds__(NT) void k_tiles(QParams p) {
    constexpr int V = BF ? 8 : 4;          // columns per thread
    const Elem E = make_elem(p.elem, p.asym);
    const int64_t vpr = p.cols / V;         // thread columns per band
    const int64_t total = (p.rows / BR) * vpr;
    const int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x;
    const bool active = q < total;
    const int64_t band = active ? q / vpr : 0;
    const int64_t c0 = active ? (q - band * vpr) * V : 0;
    const int64_t r0 = band * BR;
    const bool two_d = p.bc > 1;
    const int G = two_d ? (BR / V > 0 ? BR / V : 1) : 1;
    const bool leader = (threadIdx.x % G) == 0;

    uint32_t w[BR][4];
#pragma unroll
    for (int rr = 0; rr < BR; rr++) {
        if (active) {
            u32x4 t = ld_stream16(static_cast<const uint8_t*>(p.x) + ((r0 + rr) * p.ld + c0) * (BF ? 2 : 4));
            w[rr][0] = t.x; w[rr][1] = t.y; w[rr][2] = t.z; w[rr][3] = t.w;
        } else {
            w[rr][0] = w[rr][1] = w[rr][2] = w[rr][3] = 0;
        }
    }

    // per column statistics over the band
    float amax[V], mn[V], mx[V];
    int fin[V];
#pragma unroll
    for (int j = 0; j < V; j++) { amax[j] = 0.f; mn[j] = INFINITY; mx[j] = -INFINITY; fin[j] = 1; }
#pragma unroll
    for (int rr = 0; rr < BR; rr++) {
#pragma unroll
        for (int j = 0; j < V; j++) {
            float v = word_elem<BF>(w[rr], j);
            if (!finitef(v)) { fin[j] = 0; continue; }
            amax[j] = fmaxf(amax[j], fabsf(v));
            mn[j] = fminf(mn[j], v);
            mx[j] = fmaxf(mx[j], v);
        }
    }
    if (two_d) {
        // one block covers all V columns of this thread and G - 1 neighbours
        float a = amax[0], lo = mn[0], hi = mx[0];
        int f = fin[0];
#pragma unroll
        for (int j = 1; j < V; j++) { a = fmaxf(a, amax[j]); lo = fminf(lo, mn[j]); hi = fmaxf(hi, mx[j]); f &= fin[j]; }
        a = group_max_rt(a, G);
        f = group_and_rt(f, G);
        if (p.asym) { lo = group_min_rt(lo, G); hi = group_max_rt(hi, G); }
#pragma unroll
        for (int j = 0; j < V; j++) { amax[j] = a; mn[j] = lo; mx[j] = hi; fin[j] = f; }
    }

    const float g = (p.scale == SC_NVFP4) ? *p.tensor_scale : 1.0f;
    const int eref = (p.scale == SC_E3M0) ? *p.ref_exp : 0;
    const bool ue5 = p.scale == SC_UE5M3;

    int kind[V], e[V], sc[V];
    float S[V], sb[V], o[V];
    uint16_t ob[V];
#pragma unroll
    for (int j = 0; j < V; j++) {
        kind[j] = 0; e[j] = 0; sc[j] = 0; S[j] = 1.f; sb[j] = 1.f; o[j] = 0.f; ob[j] = 0;
        if (!fin[j]) {
            kind[j] = 3;
            sc[j] = (p.scale == SC_UE4M3 || p.scale == SC_NVFP4) ? 0x7f : 0xff;
        } else if (p.asym) {
            if (E.kind == INT4) {
                ob[j] = bf16_floor(mn[j]);
                o[j] = bf16f(ob[j]);
                float R = mx[j] - o[j];
                e[j] = R > 0.f ? e8m0_exp(p.rule, p.tau, E, R) : -127;
            } else {
                // the mid-range, each end halved first so that it cannot overflow
                ob[j] = bf16_rne(mx[j] * 0.5f + mn[j] * 0.5f);
                o[j] = bf16f(ob[j]);
            }
        } else if (p.scale == SC_E8M0) {
            e[j] = e8m0_exp(p.rule, p.tau, E, amax[j]);
        } else if (p.scale == SC_E3M0) {
            int cdown = 7;
            if (amax[j] > 0.f) {
                cdown = eref - e_ceil(amax[j], E.qmax);
                cdown = cdown < 0 ? 0 : (cdown > 7 ? 7 : cdown);
            }
            e[j] = eref - cdown;
            sc[j] = cdown;
        } else {
            float t = amax[j] / E.qmax;
            if (p.scale == SC_NVFP4) t = t / g;
            sc[j] = fp8_code(ue5, t);
            sb[j] = fp8_value(ue5, sc[j]);
            S[j] = (p.scale == SC_NVFP4) ? sb[j] * g : sb[j];
            kind[j] = (S[j] == 0.f) ? 2 : 1;
        }
    }
    if (p.asym && E.kind != INT4) {
        // E2M1 with offset: the exponent comes from max |x - o| over the block
        float ym[V];
#pragma unroll
        for (int j = 0; j < V; j++) ym[j] = 0.f;
#pragma unroll
        for (int rr = 0; rr < BR; rr++)
#pragma unroll
            for (int j = 0; j < V; j++) ym[j] = fmaxf(ym[j], fabsf(word_elem<BF>(w[rr], j) - o[j]));
        if (two_d) {
            float a = ym[0];
#pragma unroll
            for (int j = 1; j < V; j++) a = fmaxf(a, ym[j]);
            a = group_max_rt(a, G);
#pragma unroll
            for (int j = 0; j < V; j++) ym[j] = a;
        }
#pragma unroll
        for (int j = 0; j < V; j++)
            if (kind[j] == 0) e[j] = e8m0_exp(p.rule, p.tau, E, ym[j]);
    }
#pragma unroll
    for (int j = 0; j < V; j++)
        if (kind[j] != 3 && (p.scale == SC_E8M0 || p.asym)) sc[j] = e[j] + 127;

    double s2 = 0, e2 = 0;
    unsigned long long nz = 0, fl = 0, zb = 0;
    int allzero[V];
#pragma unroll
    for (int j = 0; j < V; j++) allzero[j] = 1;
    const int64_t crow = (E.bits == 4) ? p.cols / 2 : p.cols * 3 / 4;

#pragma unroll
    for (int rr = 0; rr < BR; rr++) {
        const int64_t r = r0 + rr;
        uint32_t rnd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (p.round == SR) {
            const uint64_t idx = (uint64_t)(r * p.cols + c0);
            draws8(p.seed, p.off, idx >> 3, rnd);
            if (!BF && (idx & 4)) {
                rnd[0] = rnd[4]; rnd[1] = rnd[5]; rnd[2] = rnd[6]; rnd[3] = rnd[7];
            }
        }
        int code[V];
        float d[V];
#pragma unroll
        for (int j = 0; j < V; j++) {
            const float xv = word_elem<BF>(w[rr], j);
            int c;
            float dv;
            if (kind[j] == 3) {
                c = 0;
                dv = __uint_as_float(0x7fc00000u);
            } else {
                float v;
                if (kind[j] == 0) v = (p.asym ? (xv - o[j]) : xv) * pow2f(-e[j]);
                else if (kind[j] == 1) v = xv / S[j];
                else v = (fbits(xv) >> 31) ? -0.f : 0.f;
                c = encode(E, kind[j] == 2 ? RTNE : p.round, v, rnd[j]);
                float val = decode(E, c);
                if (kind[j] == 0) {
                    dv = val * pow2f(e[j]);
                    if (p.asym) dv = dv + o[j];
                } else {
                    dv = val * sb[j];
                    if (p.scale == SC_NVFP4) dv = dv * g;
                }
            }
            code[j] = c;
            d[j] = dv;
            allzero[j] &= (dv == 0.f);
            if (active && p.parts) {
                double xd = xv, dd = dv;
                s2 += xd * xd;
                e2 += (xd - dd) * (xd - dd);
                nz += (xv != 0.f);
                fl += (xv != 0.f && dv == 0.f);
            }
        }
        if (active) {
            uint8_t* row = p.codes + r * crow;
            if (E.bits == 4) {
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < V; j++) word |= (uint32_t)code[j] << (4 * j);
                if (V == 8) *reinterpret_cast<uint32_t*>(row + c0 / 2) = word;
                else *reinterpret_cast<uint16_t*>(row + c0 / 2) = (uint16_t)word;
            } else {
                uint64_t bitsw = 0;
#pragma unroll
                for (int j = 0; j < V; j++) bitsw |= (uint64_t)code[j] << (6 * j);
                uint8_t* dst = row + c0 * 3 / 4;
                if (V == 8) {
                    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
                    d16[0] = (uint16_t)bitsw; d16[1] = (uint16_t)(bitsw >> 16); d16[2] = (uint16_t)(bitsw >> 32);
                } else {
                    dst[0] = (uint8_t)bitsw; dst[1] = (uint8_t)(bitsw >> 8); dst[2] = (uint8_t)(bitsw >> 16);
                }
            }
            if (p.dq) {
                if (p.dq_bf16) {
                    uint16_t* dst = static_cast<uint16_t*>(p.dq) + r * p.cols + c0;
#pragma unroll
                    for (int j = 0; j < V; j++) dst[j] = bf16_rne(d[j]);
                } else {
                    float* dst = static_cast<float*>(p.dq) + r * p.cols + c0;
#pragma unroll
                    for (int j = 0; j < V; j++) dst[j] = d[j];
                }
            }
        }
    }

    // scales (and offsets): column blocks: V bytes per band row; 2D: one per block
    if (two_d) {
        int az = allzero[0];
#pragma unroll
        for (int j = 1; j < V; j++) az &= allzero[j];
        az = group_and_rt(az, G);
        if (active && leader) {
            const int64_t sidx = band * (p.cols / BR) + c0 / BR;
            p.scales[sidx] = (uint8_t)sc[0];
            if (p.asym) p.offsets[sidx] = kind[0] == 3 ? (uint16_t)0 : ob[0];
            zb += (unsigned long long)az;
        }
    } else if (active) {
#pragma unroll
        for (int j = 0; j < V; j++) {
            const int64_t sidx = band * p.cols + c0 + j;
            p.scales[sidx] = (uint8_t)sc[j];
            if (p.asym) p.offsets[sidx] = kind[j] == 3 ? (uint16_t)0 : ob[j];
            zb += (unsigned long long)allzero[j];
        }
    }
    if (p.parts) block_stats<NT>(s2, e2, nz, fl, zb, p.parts + blockIdx.x);
}

}  // namespace

int64_t tiles_grid(const QParams& p) {
    const int V = p.in_bf16 ? 8 : 4;
    return ((p.rows / p.br) * (p.cols / V) + NT - 1) / NT;
}

hipError_t launch_tiles(const QParams& p, hipStream_t s) {
    const int64_t grid = tiles_grid(p);
    if (grid == 0) return hipSuccess;
#define MX_TILE_CASE(BFv, BRv) \
    if (p.in_bf16 == (BFv) && p.br == (BRv)) { k_tiles<BFv, BRv><<<grid, NT, 0, s>>>(p); return hipGetLastError(); }
    MX_TILE_CASE(true, 8) MX_TILE_CASE(true, 16) MX_TILE_CASE(true, 32)
    MX_TILE_CASE(false, 8) MX_TILE_CASE(false, 16) MX_TILE_CASE(false, 32)
#undef MX_TILE_CASE
    return hipErrorInvalidValue;
}

}  // namespace mxk
