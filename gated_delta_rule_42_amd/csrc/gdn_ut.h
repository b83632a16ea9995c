// The UT transform of one 64-token chunk on the first four waves of a work-group: T = (I + A)^{-1} for a
// strictly lower triangular A (so I + A is unit lower triangular and needs no pivoting).
#pragma once

#include "gdn_device.h"

namespace gdn {

// Block (IB, JB) of T below the block diagonal: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj, fp32
// MFMA (16x16x4). It reads the diagonal block T_ii and the blocks above it in its own column.
// All operands of the block are read before the products, so the reads overlap instead of
// each product waiting for its own.
template <int PF, int IB, int JB>
__device__ __forceinline__ void ut_block(const float* At, float* Tt, int lane) {
    constexpr int D = IB - JB;
    const int l16 = lane & 15, lq = lane >> 4;
    {
        constexpr int ib = IB, jb = JB;
        float av[4 * D], bv[4 * D], tv[4];
#pragma unroll
        for (int mm = 0; mm < D; ++mm)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int m = jb + mm;
                av[4 * mm + s] = At[(16 * ib + l16) * PF + 16 * m + 4 * s + lq];
                bv[4 * mm + s] = Tt[(16 * m + 4 * s + lq) * PF + 16 * jb + l16];
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) tv[s] = Tt[(16 * ib + l16) * PF + 16 * ib + 4 * lq + s];
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4 * D; ++k) z = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k], bv[k], z, 0, 0, 0);
        // z is in accumulator layout (lane holds rows 4*lq+s of column l16); use it as the
        // right operand with k relabelled to 4*lq + s in step s.
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) t = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[s], z[s], t, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) Tt[(16 * ib + 4 * lq + v) * PF + 16 * jb + l16] = -t[v];
    }
}

// A and T are fp32 [64, PF] in LDS (row pitch PF); A's strictly lower part is read, T's lower
// blocks are written (blocks above the 16x16 block diagonal are left untouched). Diagonal
// 16x16 blocks: wave w inverts block w by forward substitution, lane l16 computing column l16
// with the block's strictly lower entries held in registers. Then, after one barrier, wave w
// walks block column w downwards (ut_block): each block needs only the diagonal blocks and the
// blocks above it in its column, which the same wave wrote just before, so no further barrier
// is needed until the end. Called by all threads of the work-group (waves past the fourth only
// take part in the barriers); ends with a barrier.
template <int PF>
__device__ __forceinline__ void ut_inverse64(const float* At, float* Tt, int wave, int lane) {
    const int l16 = lane & 15, lq = lane >> 4;
    if (wave < 4) {
        const float* Ab = At + 16 * wave * PF + 16 * wave;
        float a[16][16];
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
            for (int i = 0; i < r; ++i) a[r][i] = Ab[r * PF + i];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc0 = (r == l16) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
            for (int i = 0; i < r; i += 2) {
                acc0 -= a[r][i] * x[i];
                if (i + 1 < r) acc1 -= a[r][i + 1] * x[i + 1];
            }
            x[r] = acc0 + acc1;
        }
        if (lq == 0) {
            float* Tb = Tt + 16 * wave * PF + 16 * wave;
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[r * PF + l16] = x[r];
        }
    }
    __syncthreads();
    switch (wave) {
        case 0:
            ut_block<PF, 1, 0>(At, Tt, lane);
            ut_block<PF, 2, 0>(At, Tt, lane);
            ut_block<PF, 3, 0>(At, Tt, lane);
            break;
        case 1:
            ut_block<PF, 2, 1>(At, Tt, lane);
            ut_block<PF, 3, 1>(At, Tt, lane);
            break;
        case 2:
            ut_block<PF, 3, 2>(At, Tt, lane);
            break;
        default:
            break;
    }
    __syncthreads();
}

}  // namespace gdn
