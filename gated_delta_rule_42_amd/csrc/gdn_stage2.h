// LDS layout of a chunk's K or Q tile and the transposed K fragment read, shared by the
// state-propagation kernels.
#pragma once

#include "gdn_device.h"

namespace gdn {

// Element offset of (row, col) in the LDS copy of K or Q. 16-bit operands with d_k = 128 use
// an unpadded 256-byte row with its 8-byte granules XOR-swizzled by the row, so that both
// ways the kernel reads K are free of bank conflicts: row fragments (16 rows x 8 bytes per
// half-wave) and transposing reads (8 rows x 32 bytes per half-wave). The swizzle keeps each
// even/odd granule pair adjacent, so 16-byte staging stores stay contiguous. Other shapes use
// a padded row.
template <typename TM, int DK>
struct KQLayout {
    static constexpr bool kSwizzle = sizeof(TM) == 2 && DK == 128;
    static constexpr int kPitch = kSwizzle ? DK : DK + 16 / (int)sizeof(TM);
    __device__ __forceinline__ static int off(int row, int col) {
        if constexpr (kSwizzle) {
            const int g = (col >> 2) ^ (4 * (row & 7) + 2 * ((row >> 3) & 1));
            return row * DK + 4 * g + (col & 3);
        } else {
            return row * kPitch + col;
        }
    }
};

// Operand fragment of K^T (rows d_k 16j + l16, k = tokens) read transposed from the LDS
// copy of K: slots 0-3 are tokens t0 + 0..3, slots 4-7 tokens t1 + 0..3 (t0, t1 multiples
// of 4). 16-bit operands use the gfx950 transposing read, lane s of each 16-lane group
// addressing row t + s/4, columns 16j + 4*(s%4) .. +3.
template <typename TM, int DK>
__device__ __forceinline__ Frag<TM> load_kt(const TM* K, int t0, int t1, int j) {
    using KL = KQLayout<TM, DK>;
    const int l16 = threadIdx.x & 15;
    if constexpr (sizeof(TM) == 2) {
        const int rr = l16 >> 2, cc = 16 * j + 4 * (l16 & 3);
        const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(K + KL::off(t0 + rr, cc)));
        const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(K + KL::off(t1 + rr, cc)));
        const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
        Frag<TM> f;
        f.v = make_uint4(ua.x, ua.y, ub.x, ub.y);
        return f;
    } else {
        const int c = 16 * j + l16;
        Frag<TM> f;
        f.lo = make_float4(K[KL::off(t0, c)], K[KL::off(t0 + 1, c)], K[KL::off(t0 + 2, c)], K[KL::off(t0 + 3, c)]);
        f.hi = make_float4(K[KL::off(t1, c)], K[KL::off(t1 + 1, c)], K[KL::off(t1 + 2, c)], K[KL::off(t1 + 3, c)]);
        return f;
    }
}

}  // namespace gdn
