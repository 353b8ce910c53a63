// gemm_cstore.hpp -- the bf16 C store path shared by the LDS-staged GEMM
// kernels: a wave's 32 x 32 accumulator tiles (lane l, register r holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32]) go through a private LDS strip of 16 rows
// and out as 16-byte row stores.
#pragma once
#include "mx_kernels.hpp"

namespace mxk {

typedef float v16f_cs __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_cs __attribute__((ext_vector_type(4)));

// one C tile's store path: bf16 rows staged per 16-row strip in a private
// LDS area of each wave (LDS operations of one wave complete in order, so the
// strips need no barrier), then written with 16-byte stores.  With `exact`,
// every wave issues exactly NSTORE buffer stores, lanes outside C aiming past
// the resource (the count matters to the in-order vector-memory waits of the
// next tile); otherwise stores are per element where a 16-byte chunk would
// cross the end of a row.
template <class G>
struct CStore {
    static constexpr int TI = G::TI, TJ = G::TJ;
    static constexpr int SROWS = 16;                 // rows per strip
    static constexpr int CROW = 64 * TJ + 16;        // padded bf16 strip row
    static constexpr int CPRC = 4 * TJ;              // 16-byte chunks per strip row
    static constexpr int RPI = 64 / CPRC;            // strip rows per wave-store
    static constexpr int NSTORE = TI * (32 / SROWS) * (SROWS / RPI);
    static constexpr int AREA = SROWS * CROW;        // LDS bytes per wave
};

template <class G, bool EXACT>
__device__ __forceinline__ void store_c_bf16(const v16f_cs (&acc)[G::TI][G::TJ], uint8_t* ct, void* C, int64_t m0,
                                             int64_t n0, int64_t M, int64_t N, int64_t ldc, int wm, int wn, int lane,
                                             int half, int lrow) {
    using S = CStore<G>;
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const int64_t vrows = M - m0 < G::BM ? M - m0 : G::BM;
    uint8_t* cbase = static_cast<uint8_t*>(C) + m0 * ldc * 2;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(cbase, (short)0, (int)(vrows * ldc * 2),
                                                                        0x00020000);
#pragma unroll
    for (int i = 0; i < S::TI; i++)
#pragma unroll
        for (int hs = 0; hs < 32 / S::SROWS; hs++) {
#pragma unroll
            for (int j = 0; j < S::TJ; j++)
#pragma unroll
                for (int r = 8 * hs; r < 8 * hs + 8; r += 2) {
                    const f2 f = {acc[i][j][r], acc[i][j][r + 1]};
                    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2));
                    const int ml = 8 * (r / 4) + 4 * half + (r % 4) - S::SROWS * hs, nl = j * 32 + lrow;
                    *reinterpret_cast<uint16_t*>(ct + ml * S::CROW + nl * 2) = (uint16_t)w;
                    *reinterpret_cast<uint16_t*>(ct + (ml + 1) * S::CROW + nl * 2) = (uint16_t)(w >> 16);
                }
#pragma unroll
            for (int q = 0; q < S::SROWS / S::RPI; q++) {
                const int row = q * S::RPI + lane / S::CPRC, chunk = lane % S::CPRC;
                const int mt = wm * 32 * S::TI + i * 32 + hs * S::SROWS + row;       // row in the tile
                const int64_t n = n0 + wn * 32 * S::TJ + chunk * 8;
                const u32x4_cs v = *reinterpret_cast<const u32x4_cs*>(ct + row * S::CROW + chunk * 16);
                if constexpr (EXACT) {
                    const int off = n < N ? (int)(mt * ldc * 2 + n * 2) : (int)0x80000000u;
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
                } else {
                    const int64_t m = m0 + mt;
                    if (m >= M || n >= N) continue;
                    uint16_t* dst = static_cast<uint16_t*>(C) + m * ldc + n;
                    if (n + 8 <= N && (ldc % 8) == 0) {
                        *reinterpret_cast<u32x4_cs*>(dst) = v;
                    } else {
#pragma unroll
                        for (int k = 0; k < 8; k++)
                            if (n + k < N) dst[k] = (uint16_t)(v[k >> 1] >> (16 * (k & 1)));
                    }
                }
            }
        }
}

}  // namespace mxk
