// LDS layouts of a chunk's operands (the K or Q tile of the register-staged kernels, the byte
// images of the DMA-fed ones) and pieces shared by the state-propagation kernels.
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

// ------------------------------------------------------- LDS images (bf16 inputs)
// For bf16 inputs stage 1 stores the fp16 operands of stage 2 (K, diag(e^gamma) Q: W = d_k
// columns; Mmat, P: W = 64) as byte images of the LDS tiles stage 2 reads, so that stage 2
// copies them with plain 1 KB DMA blocks. A row is cut into 16-byte pieces; piece pc holds
// the 8 contraction indices one lane feeds to a 16x16x32 product, columns
// 32(pc>>2) + 4(pc&3) + 0..3 then the same + 16, and sits at position pc ^ img_swz<W>(r)
// of row r. LDS serves a 16-byte read 8 lanes (128 bytes) at a time and an 8-byte read 16 lanes
// at a time; the permutation is chosen so that the 8 rows of a row-fragment read (W = 128: one
// row per 256 bytes, so only the position within the row can separate them) fall on 8 distinct
// 16-byte positions modulo 128, and so that the transposing reads of K (4 rows x 32 bytes per
// 16 lanes) meet the least bank sharing their shape allows (they are read as 8-byte halves of
// 16-byte positions, so 16 lanes can use at most 8 of the 16 half-positions in 128 bytes).
template <int W>
__device__ __forceinline__ int img_swz(int r) {
    if constexpr (W == 128) return (4 * (r & 3) + ((r >> 2) & 3)) ^ (r & 2);
    else return (r >> 1) & 7;  // W = 64: two rows per 256 bytes
}
// element offset, in a [64, W] image, of the 4-element run at column c (c % 4 == 0) of row r
template <int W>
__device__ __forceinline__ int img_off(int r, int c) {
    const int s = c >> 5, a = (c >> 4) & 1, m = (c >> 2) & 3;
    return r * W + 8 * ((4 * s + m) ^ img_swz<W>(r)) + 4 * a;
}
// source columns of image piece i (pieces numbered in storage order): c0 .. c0+3, c0+16 .. c0+19
template <int W>
__device__ __forceinline__ void img_piece(int i, int& r, int& c0) {
    constexpr int NP = W / 8;
    r = i / NP;
    const int pc = (i % NP) ^ img_swz<W>(r);
    c0 = 32 * (pc >> 2) + 4 * (pc & 3);
}

// ----------------------------------------------- DMA-fed stage 2: shared pieces
// Output staging for one chunk: the compute waves leave o^T tiles here and the store wave
// writes them out as whole rows of the work-group's columns. Rows are padded by 16 bytes so
// that the compute waves' 4-column writes of 16 consecutive tokens fall in distinct banks.
template <typename TO, int DVT>
struct alignas(16) OStage {
    static constexpr int ROWB = DVT * (int)sizeof(TO);  // bytes of one token's columns
    static constexpr int PITCH = ROWB + 16;
    char b[64 * PITCH];
};

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Work-group barrier that orders LDS accesses only: the waves' global stores and copies are
// not waited for (the DMA wave waits for its own copies explicitly).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same without the fences, whose release half makes the compiler wait for every outstanding
// vector memory operation of the wave, global loads and stores included: this barrier waits for
// the wave's LDS accesses only and keeps the compiler from moving memory accesses across it. For
// waves that copy nothing into LDS (their global loads are waited for where used), or that wait
// for their copies into LDS themselves, with explicit counts, before it.
__device__ __forceinline__ void lds_barrier_lgkm() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The ordered walk of the long-chain split accepts segment g >= 1 when the second pass fixed it
// (counts[g] < its chunk count) and ends at the first segment with no chunks. This returns the
// first g >= 1 where the walk stops accepting, because segment g is empty or was not fixed, or
// seg_n when there is none: every lane tests one segment, 64 per step, so that a walk over
// segments that were all fixed reads the counts once instead of one dependent load per segment.
// chunks_of(g) gives segment g's chunk count; the result is uniform over the wave.
template <typename F>
__device__ __forceinline__ int walk_first_stop(const int* counts, int seg_n, F chunks_of) {
    const int lane = (int)(threadIdx.x & 63);
    for (int base = 1; base < seg_n; base += 64) {
        const int g = base + lane;
        bool stop = false;
        if (g < seg_n) {
            const long len = chunks_of(g);
            stop = len == 0 || counts[g] >= len;
        }
        const unsigned long long m = __builtin_amdgcn_ballot_w64(stop);
        if (m) return base + (int)__builtin_ctzll(m);
    }
    return seg_n;
}

}  // namespace gdn
