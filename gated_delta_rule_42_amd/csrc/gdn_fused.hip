// Chunkwise forward pass of the gated delta rule for bf16 inputs with d_k = d_v = 128, in one
// kernel: the chunk-local operators of the WY representation carrying the gate (paper note
// "Gated Delta Networks: Improving Mamba2 with Delta Rule", mechanism paragraph; record
// "LIT-137", "Standing in the anthology") are built in LDS by the same work-group that carries
// the state, one chunk ahead of it, so they never travel through HBM: per chunk-head the kernel
// reads q, k, v, g, beta and writes o, about 64 KB, where the two-stage path moves 161 KB.
//
// One work-group per (sequence, head) (or per segment of one, see SEG below), eight waves in two
// roles that run side by side, one of each per SIMD:
//   * state waves 0-3: wave w owns d_v columns 32w .. 32w+31 (lane column l16 of half hh is
//     32w + 2 l16 + hh, so a lane's two columns are adjacent) with the fp32 state S^T [d_k, 32]
//     in registers, and steps chunk c: X = K S^T, R = V - diag(e^gamma) X, Delta = Mmat R,
//     O^T = diag(e^gamma) S Q^T + Delta^T P^T stored to global memory, then
//     S^T <- e^{gamma_last} S^T + K^T diag(e^{gamma_last - gamma}) Delta;
//   * operator waves 4-7 (u = wave - 4) build chunk c+1's operators in the other LDS slot, each
//     from its quarter of the chunk's rows, loaded whole-row (coalesced) one phase ahead:
//     A1: the fp16 images of K and Q rows 16u .. 16u+15, those V rows, the in-chunk scan of g;
//     A2: the gated Gram blocks of row u of A = strict_lower(diag(beta) K K^T * Gamma) and
//         row 3-u of P = (Q K^T) * Gamma * [i <= r] from the images (five 16x16 blocks per
//         wave, fp16 matrix core: bf16 values are exact in fp16), and T's diagonal block
//         (I + A_uu)^{-1} by forward substitution;
//     C:  Mmat's diagonal block u and one of T's lower-left blocks per wave on the fp32 matrix
//         core, from T_IJ = -T_II sum_{m=J}^{I-1} A_Im T_mJ (each wave recomputes the blocks its
//         own needs, so no wave waits for another), with its Mmat block.
// Three work-group barriers per chunk separate the phases. The state waves form R, Delta and O of
// chunk c in A1, and in A2 update the state with chunk c and then form X = K S^T and S Q^T of
// chunk c+1 (from the images the operator waves wrote in A1); their phase C is empty.
// Every gate factor is exp of a non-positive number: below the 16x16 diagonal blocks the factor
// exp(gamma_r - gamma_i) is taken as exp(gamma_r - gamma_m) exp(gamma_m - gamma_i) with m the last
// row of the column block, inside them one exp per entry of the masked, clamped difference.
//
// Long chains are cut into segments as in the two-stage path (SEG = 1: every segment at once,
// from h0 or zero, with state records; SEG = 2: every segment g >= 1 again from the final state
// SEG = 1 left for g-1, up to the first record its state equals bit for bit; SEG = 3: the ordered
// walk that accepts the reruns that started from the true state and redoes the rest). o and hT
// equal those of the unsplit kernel bit for bit.
#include <cstdlib>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_stage2.h"

namespace gdn {

namespace {

constexpr int FD = 128;            // d_k = d_v
constexpr int NSW = 4;             // state waves, 32 d_v columns each
constexpr int NOW = 4;             // operator waves
constexpr int FNT = (NSW + NOW) * 64;
constexpr int NKB = FD / 16;       // 16-row d_k tiles of the state
constexpr int NKS = FD / 32;       // 32-wide d_k slices

// One chunk's operators as the state waves read them (the layouts of img_off).
struct alignas(16) FSlot {
    _Float16 Q[64 * FD];   // Q, unscaled (bf16 values are exact in fp16's normal range)
    _Float16 K[64 * FD];
    _Float16 M[64 * 64];   // Mmat = T diag(beta)
    _Float16 P[64 * 64];   // (Q K^T) * exp(gamma_r - gamma_i) * [i <= r]
    float eg[64];          // e^{gamma_r}
    float ed[64];          // e^{gamma_last - gamma_r}
};
// A chunk's V rows (bf16).
struct alignas(16) FV {
    uint16_t v[64 * FD];
};

// The operator waves' working set: 16x16 fp32 blocks, rows padded to kBP floats.
constexpr int kBP = 20;
constexpr int kBlk = 16 * kBP;
struct alignas(16) FOps {
    float A[10 * kBlk];    // block (I, J) at I(I+1)/2 + J: rows of A_IJ (J < I), A_II transposed
    float D[4 * kBlk];     // T's diagonal blocks (I + A_II)^{-1}, rows
    float gam[NOW][64];    // each operator wave's own copy of the chunk's gamma and beta
    float beta[NOW][64];
    __device__ __forceinline__ float* a(int I, int J) { return A + (I * (I + 1) / 2 + J) * kBlk; }
    __device__ __forceinline__ float* d(int I) { return D + I * kBlk; }
};

// Raw bf16 rows 16U .. 16U+15 of one chunk's K, Q and V as operator wave U loads them: load e
// holds row 16U + 4e + lane/16, columns 8 (lane % 16) .. +7; and g, beta (lane = token). Rows
// past the chunk's end read as zeros.
struct ORaw {
    u32x4_t k[4], q[4], v[4];
    float g, b;
};

// The loads take the lane's row and column as their vector offset and the rows' block as their
// scalar offset, so that no per-load address lives in a vector register across the chunk loop.
template <int U>
__device__ __forceinline__ void oraw_load(ORaw& r, const ChunkProblem& p, long bos, int len, int h, int lane) {
    const int H = p.H;
    const unsigned bytes = (unsigned)((len - 1) * H * FD + FD) * 2;
    const long base = (bos * H + h) * FD;
    const auto kr = make_rsrc(static_cast<const uint16_t*>(p.k) + base, bytes);
    const auto qr = make_rsrc(static_cast<const uint16_t*>(p.q) + base, bytes);
    const auto vr = make_rsrc(static_cast<const uint16_t*>(p.v) + base, bytes);
    const int voff = (lane >> 4) * H * FD * 2 + 16 * (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int so = (16 * U + 4 * e) * H * FD * 2;
        r.k[e] = __builtin_amdgcn_raw_buffer_load_b128(kr, voff, so, 0);
        r.q[e] = __builtin_amdgcn_raw_buffer_load_b128(qr, voff, so, 0);
        r.v[e] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff, so, 0);
    }
    r.g = 0.f;
    r.b = 0.f;
    if (lane < len) {
        const long o = (bos + lane) * H + h;
        r.g = p.g[o];
        r.b = p.beta[o];
    }
}

// One row piece of an fp16 image from the lane's 8 raw columns 8c' .. 8c'+7 (c' = lane % 16):
// a piece holds the 4-column runs 8s + m and 8s + 4 + m of its row (s = c' / 4, m = 0..3); the
// lanes c' and c' ^ 2 hold each other's second run and trade it (one DPP exchange per dword).
// Returns the piece and its first column 32s + 4m.
__device__ __forceinline__ uint4 image_piece(const u32x4_t& x, int lane, int& c0) {
    const int cp = lane & 15, j = cp & 3;
    const bool lo = j < 2;
    const uint32_t s0 = lo ? x[2] : x[0], s1 = lo ? x[3] : x[1];
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x4E, 0xF, 0xF, false);
    const uint32_t w0 = lo ? x[0] : r0, w1 = lo ? x[1] : r1, w2 = lo ? r0 : x[2], w3 = lo ? r1 : x[3];
    c0 = 32 * (cp >> 2) + 4 * (((j & 1) << 1) | (j >> 1));
    auto cv = [](uint32_t w) { return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)); };
    return make_uint4(cv(w0), cv(w1), cv(w2), cv(w3));
}

// Gate factors exp(gamma_r - gamma_i) of block (I, J) for the lane's row r = 16I + l16 and
// columns i = 16J + 4lq + 0..3, masked to i < r (INCL: i <= r) inside the diagonal block.
template <bool INCL>
__device__ __forceinline__ void gate_row(int I, int J, const float* gam, int l16, int lq, float (&f)[4]) {
    const int r = 16 * I + l16;
    const float gr = gam[r];
    const float4 gi = *reinterpret_cast<const float4*>(&gam[16 * J + 4 * lq]);
    const float giv[4] = {gi.x, gi.y, gi.z, gi.w};
    if (I == J) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * J + 4 * lq + v;
            const float e = __expf(fminf(gr - giv[v], 0.f));
            f[v] = (i < r || (INCL && i == r)) ? e : 0.f;
        }
    } else {
        const float gm = gam[16 * J + 15];
        const float rowf = __expf(fminf(gr - gm, 0.f));
#pragma unroll
        for (int v = 0; v < 4; ++v) f[v] = rowf * __expf(fminf(gm - giv[v], 0.f));
    }
}

// Phase A1 of operator wave U: its rows of the K and Q images and of V, the gate tables.
template <int U>
__device__ __forceinline__ void op_a1(FSlot& d, FV& dv, FOps& ops, const ORaw& r, int lane) {
    const int rsub = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = 16 * U + 4 * e + rsub;
        int c0;
        const uint4 kp = image_piece(r.k[e], lane, c0);
        *reinterpret_cast<uint4*>(&d.K[img_off<FD>(row, c0)]) = kp;
        const uint4 qp = image_piece(r.q[e], lane, c0);
        *reinterpret_cast<uint4*>(&d.Q[img_off<FD>(row, c0)]) = qp;
        *reinterpret_cast<u32x4_t*>(&dv.v[row * FD + 8 * (lane & 15)]) = r.v[e];
    }
    const float x = wave_inclusive_sum(r.g);
    ops.gam[U][lane] = x;
    ops.beta[U][lane] = r.b;
    if constexpr (U == 0) {
        const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
        d.eg[lane] = __expf(x);
        d.ed[lane] = __expf(last - x);
    }
}

// Phase A2 of operator wave U: the Gram blocks of A row U (blocks (U, J), J <= U) and P row
// 3-U (blocks (3-U, J), J <= 3-U), gated, and T's diagonal block U (into the rows of ops.d(U)).
// Lane: row 16I + l16, columns 16J + 4lq + 0..3 (the diagonal block of A: transposed).
template <int U>
__device__ __forceinline__ void op_a2(FSlot& d, FOps& ops, int lane) {
    const int l16 = lane & 15, lq = lane >> 4;
    constexpr int PI = 3 - U;
    constexpr int KM = U > PI ? U : PI;   // K row blocks 0 .. KM are needed
    const float* gam = ops.gam[U];
    const float* beta = ops.beta[U];
    f32x4_t ga[U + 1], gp[PI + 1];
#pragma unroll
    for (int J = 0; J <= U; ++J) ga[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= PI; ++J) gp[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        uint4 kf[KM + 1];
#pragma unroll
        for (int J = 0; J <= KM; ++J) kf[J] = *reinterpret_cast<const uint4*>(&d.K[img_off<FD>(16 * J + l16, 32 * s + 4 * lq)]);
        const uint4 qf = *reinterpret_cast<const uint4*>(&d.Q[img_off<FD>(16 * PI + l16, 32 * s + 4 * lq)]);
#pragma unroll
        for (int J = 0; J <= U; ++J) ga[J] = mfma_f16(kf[J], kf[U], ga[J]);
#pragma unroll
        for (int J = 0; J <= PI; ++J) gp[J] = mfma_f16(kf[J], qf, gp[J]);
    }
    // A below the diagonal block, P
#pragma unroll
    for (int J = 0; J < U; ++J) {
        float f[4];
        gate_row<false>(U, J, gam, l16, lq, f);
        const float br = beta[16 * U + l16];
        *reinterpret_cast<float4*>(&ops.a(U, J)[l16 * kBP + 4 * lq]) =
            make_float4(br * ga[J][0] * f[0], br * ga[J][1] * f[1], br * ga[J][2] * f[2], br * ga[J][3] * f[3]);
    }
#pragma unroll
    for (int J = 0; J <= PI; ++J) {
        float f[4];
        gate_row<true>(PI, J, gam, l16, lq, f);
        *reinterpret_cast<uint2*>(&d.P[img_off<64>(16 * PI + l16, 16 * J + 4 * lq)]) =
            make_uint2(pack_f16x2(gp[J][0] * f[0], gp[J][1] * f[1]), pack_f16x2(gp[J][2] * f[2], gp[J][3] * f[3]));
    }
    // A_UU transposed: the lane holds K K^T rows 16U + 4lq + v of column 16U + l16 (the Gram
    // matrix is symmetric), i.e. A[r][i] for r = 16U + 4lq + v, i = 16U + l16
    float* At = ops.a(U, U);
    {
        const int i = 16 * U + l16;
        const float gi = gam[i];
        const float4 gr = *reinterpret_cast<const float4*>(&gam[16 * U + 4 * lq]);
        const float4 br = *reinterpret_cast<const float4*>(&beta[16 * U + 4 * lq]);
        const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, brv[4] = {br.x, br.y, br.z, br.w};
        float a[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rr = 16 * U + 4 * lq + v;
            a[v] = i < rr ? brv[v] * ga[U][v] * __expf(fminf(grv[v] - gi, 0.f)) : 0.f;
        }
        *reinterpret_cast<float4*>(&At[l16 * kBP + 4 * lq]) = make_float4(a[0], a[1], a[2], a[3]);
    }
    // T_UU = (I + A_UU)^{-1}, column c = l16 in every lane group: x = e_c, then for i = 0 .. 14
    // x[r] -= A[r][i] x[i] for r > i (column i of A is row i of the transposed block, read two
    // steps before its use)
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = rr == l16 ? 1.f : 0.f;
    float4 row[3][4];
    auto load_row = [&](int i, float4 (&b)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = (i + 1) / 4; q < 4; ++q) b[q] = *reinterpret_cast<const float4*>(&At[i * kBP + 4 * q]);
    };
    load_row(0, row[0]);
    load_row(1, row[1]);
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        if (i + 2 < 15) load_row(i + 2, row[(i + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rr = i + 1; rr < 16; ++rr) {
            const float4 v4 = row[i % 3][rr >> 2];
            const float a = (rr & 3) == 0 ? v4.x : (rr & 3) == 1 ? v4.y : (rr & 3) == 2 ? v4.z : v4.w;
            x[rr] -= a * x[i];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (lq == 0) {
        float* Dp = ops.d(U);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Dp[rr * kBP + l16] = x[rr];
    }
}

// 16x16 fp32 products on the matrix core. acc layout: the lane holds rows 4lq + 0..3 of column
// l16. prod(X, Y, acc) = acc + X Y with X read as rows from LDS and Y in acc layout (step s
// contracts k = 4lq + s).
__device__ __forceinline__ f32x4_t prod(const float* X, const f32x4_t& Y, f32x4_t acc, int l16, int lq) {
    const float4 x = *reinterpret_cast<const float4*>(&X[l16 * kBP + 4 * lq]);
    acc = mfma4(x.x, Y[0], acc);
    acc = mfma4(x.y, Y[1], acc);
    acc = mfma4(x.z, Y[2], acc);
    return mfma4(x.w, Y[3], acc);
}
__device__ __forceinline__ f32x4_t rows_to_acc(const float* Y, int l16, int lq) {
    return f32x4_t{Y[(4 * lq) * kBP + l16], Y[(4 * lq + 1) * kBP + l16], Y[(4 * lq + 2) * kBP + l16],
                   Y[(4 * lq + 3) * kBP + l16]};
}
__device__ __forceinline__ f32x4_t neg_prod(const float* X, const f32x4_t& Y, int l16, int lq) {
    return -prod(X, Y, f32x4_t{0.f, 0.f, 0.f, 0.f}, l16, lq);
}
// Mmat block (I, J) = T_IJ diag(beta) into the image, T_IJ in acc layout
template <int I, int J>
__device__ __forceinline__ void put_m(FSlot& d, const float* beta, const f32x4_t& t, int l16, int lq) {
    const float bc = beta[16 * J + l16];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        d.M[img_off<64>(16 * I + 4 * lq + v, 16 * J + (l16 & ~3)) + (l16 & 3)] = (_Float16)(t[v] * bc);
}

// Phase C of operator wave U: Mmat's diagonal block U, T's lower-left blocks and their Mmat blocks
//   U = 0: T10, T20     U = 1: T21, T32     U = 2: T30 (recomputing T10, T20)     U = 3: T31 (and T21)
template <int U>
__device__ __forceinline__ void op_c(FSlot& d, FOps& ops, int lane) {
    const int l16 = lane & 15, lq = lane >> 4;
    const float* beta = ops.beta[U];
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    {   // Mmat's diagonal block U (lane: row 16U + l16, columns 16U + 4lq + 0..3)
        const float4 t = *reinterpret_cast<const float4*>(&ops.d(U)[l16 * kBP + 4 * lq]);
        const float4 b = *reinterpret_cast<const float4*>(&beta[16 * U + 4 * lq]);
        *reinterpret_cast<uint2*>(&d.M[img_off<64>(16 * U + l16, 16 * U + 4 * lq)]) =
            make_uint2(pack_f16x2(t.x * b.x, t.y * b.y), pack_f16x2(t.z * b.z, t.w * b.w));
    }
    if constexpr (U == 0 || U == 2) {
        const f32x4_t D0 = rows_to_acc(ops.d(0), l16, lq);
        const f32x4_t T10 = neg_prod(ops.d(1), prod(ops.a(1, 0), D0, z, l16, lq), l16, lq);
        const f32x4_t T20 = neg_prod(ops.d(2), prod(ops.a(2, 1), T10, prod(ops.a(2, 0), D0, z, l16, lq), l16, lq), l16, lq);
        if constexpr (U == 0) {
            put_m<1, 0>(d, beta, T10, l16, lq);
            put_m<2, 0>(d, beta, T20, l16, lq);
        } else {
            f32x4_t s = prod(ops.a(3, 0), D0, z, l16, lq);
            s = prod(ops.a(3, 1), T10, s, l16, lq);
            s = prod(ops.a(3, 2), T20, s, l16, lq);
            put_m<3, 0>(d, beta, neg_prod(ops.d(3), s, l16, lq), l16, lq);
        }
    } else {
        const f32x4_t D1 = rows_to_acc(ops.d(1), l16, lq);
        const f32x4_t T21 = neg_prod(ops.d(2), prod(ops.a(2, 1), D1, z, l16, lq), l16, lq);
        if constexpr (U == 1) {
            put_m<2, 1>(d, beta, T21, l16, lq);
            const f32x4_t D2 = rows_to_acc(ops.d(2), l16, lq);
            put_m<3, 2>(d, beta, neg_prod(ops.d(3), prod(ops.a(3, 2), D2, z, l16, lq), l16, lq), l16, lq);
        } else {
            f32x4_t s = prod(ops.a(3, 1), D1, z, l16, lq);
            s = prod(ops.a(3, 2), T21, s, l16, lq);
            put_m<3, 1>(d, beta, neg_prod(ops.d(3), s, l16, lq), l16, lq);
        }
    }
}

// Eight consecutive values (a[0], b[0], a[1], b[1], ..) stored as T (bf16: 16 bytes, fp32: 32).
template <typename T>
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, const f32x4_t& a, const f32x4_t& b);
template <>
__device__ __forceinline__ void buf_store8<uint16_t>(__amdgpu_buffer_rsrc_t r, int off, const f32x4_t& a, const f32x4_t& b) {
    const u32x4_t v = {pack_bf16x2(a[0], b[0]), pack_bf16x2(a[1], b[1]), pack_bf16x2(a[2], b[2]), pack_bf16x2(a[3], b[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
template <>
__device__ __forceinline__ void buf_store8<float>(__amdgpu_buffer_rsrc_t r, int off, const f32x4_t& a, const f32x4_t& b) {
    const u32x4_t v0 = {__float_as_uint(a[0]), __float_as_uint(b[0]), __float_as_uint(a[1]), __float_as_uint(b[1])};
    const u32x4_t v1 = {__float_as_uint(a[2]), __float_as_uint(b[2]), __float_as_uint(a[3]), __float_as_uint(b[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v0, r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(v1, r, off + 16, 0, 0);
}

}  // namespace

template <typename TO, int SEG>
__global__ __launch_bounds__(FNT) void chunk_fused_kernel(ChunkProblem p) {
    constexpr bool CMP = SEG >= 2;
    __shared__ FSlot slot[2];       // chunk j's operators in slot[j % 2]
    __shared__ FV vb[2];            // and its V rows in vb[j % 2]
    __shared__ FOps ops;
    __shared__ int match[2][NSW];   // SEG >= 2: per state wave, state equal to the record (by chunk parity)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H;

    const long NP = (long)p.N * H;
    const long unit = blockIdx.x;
    // (sequence, head) pair in index order: this path runs no chunk-table kernel, so it takes no
    // chain order from the workspace
    const long pair = SEG == 1 ? unit / p.seg_n : SEG == 2 ? unit / (p.seg_n - 1) : unit;
    const int seg = SEG == 1 ? (int)(unit % p.seg_n) : SEG == 2 ? 1 + (int)(unit % (p.seg_n - 1)) : 0;
    const int n = (int)(pair / H), h = (int)(pair % H);

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    const long nchunks = (seos - sbos + kChunk - 1) / kChunk;
    auto chunk_len = [&](long jc) {
        const long l = seos - (sbos + jc * kChunk);
        return (int)(l < kChunk ? l : kChunk);
    };
    auto seg_range = [&](int g, long& c0, long& len) {
        c0 = (long)g * p.seg_len;
        len = max(0L, min((long)p.seg_len, nchunks - c0));
    };
    long c_first = 0, c_count = nchunks;
    if constexpr (SEG == 1 || SEG == 2) {
        seg_range(seg, c_first, c_count);
        if (seg > 0 && c_count == 0) return;   // the whole work-group leaves
    }
    const int nslot = p.seg_ncp + 2;
    auto seg_state = [&](int g, int slot) { return p.segst + ((pair * p.seg_n + g) * nslot + slot) * (long)FD * FD; };
    // chunks SEG = 2 computed per segment, in every 64-column tile's entry of the diagnostic region
    int* reran = reinterpret_cast<int*>(p.segst + NP * p.seg_n * nslot * (long)FD * FD) + pair * (FD / 64) * p.seg_n;
    auto recorded = [](int o, long len) { return o < len && (o & (o - 1)) == 0; };

    // the images' blocks above the block diagonal (Mmat, P) are never written: zero them once
    for (int i = tid; i < 64 * 64 / 8; i += FNT) {
        reinterpret_cast<uint4*>(slot[0].M)[i] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4*>(slot[0].P)[i] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4*>(slot[1].M)[i] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4*>(slot[1].P)[i] = make_uint4(0, 0, 0, 0);
    }
    lds_barrier_lgkm();

    // A range ends at the barrier after its last chunk, or (SEG >= 2) at the barrier after a chunk
    // whose end state matched the record; all waves read the same flags after the same barrier.
    auto range_done = [&](int i, long len) __attribute__((always_inline)) {
        if (i == len) return true;
        if constexpr (CMP) {
            if (i > 0) {
                bool all = true;
#pragma unroll
                for (int w = 0; w < NSW; ++w) all = all && match[(i - 1) & 1][w] != 0;
                return all;
            }
        }
        return false;
    };

    // Both roles run the same barriers: per range two before the loop (chunk c0's phases A1 and
    // A2), then per chunk i: B0 (chunk i's operators complete; the range may end here), B1, B2.
    if (wave < NSW) {
        // ------------------------------------------------------------------ state waves
        // (lane-dependent offsets are taken from opaque(lane) where used, see opaque)
        const int w = wave;
        f32x4_t ST[2][NKB];   // S^T rows 16j + 4lq + 0..3 of column 32w + 2 l16 + hh
        auto scol = [&](int hh, int ln) { return (long)(32 * w + 2 * (ln & 15) + hh) * FD + 4 * (ln >> 4); };
        auto load_state = [&](const float* src) {
            const int ln = opaque(lane);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int j = 0; j < NKB; ++j) {
                    const float4 x = *reinterpret_cast<const float4*>(src + scol(hh, ln) + 16 * j);
                    ST[hh][j] = f32x4_t{x.x, x.y, x.z, x.w};
                }
        };
        auto store_state = [&](float* dst) {
            const int ln = opaque(lane);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int j = 0; j < NKB; ++j)
                    *reinterpret_cast<float4*>(dst + scol(hh, ln) + 16 * j) =
                        make_float4(ST[hh][j][0], ST[hh][j][1], ST[hh][j][2], ST[hh][j][3]);
        };
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < NKB; ++j) ST[hh][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (SEG == 2) load_state(seg_state(seg - 1, p.seg_ncp));
        else if (SEG != 3 && p.h0 && seg == 0) load_state(p.h0 + pair * FD * FD);

        f32x4_t X[4][2], Y[4][2];   // of the next chunk, from the end of one chunk's step to the next
        f32x4_t Dl[4][2];           // Delta, from R to the state update

        // X = K S^T [64 tokens x 32 columns] and Y^T = S Q^T
        auto step_a1 = [&](const FSlot& cs) __attribute__((always_inline)) {
            const int ln = opaque(lane), l16 = ln & 15, lq = ln >> 4;
            uint4 BS[2][NKS];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int s = 0; s < NKS; ++s) BS[hh][s] = pack_f16_frag(ST[hh][2 * s], ST[hh][2 * s + 1]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    X[t][hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    Y[t][hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            uint4 KF[2][4], QF[2][4];
            auto load_kq = [&](int s, uint4 (&kf)[4], uint4 (&qf)[4]) __attribute__((always_inline)) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    kf[t] = *reinterpret_cast<const uint4*>(&cs.K[img_off<FD>(16 * t + l16, 32 * s + 4 * lq)]);
                    qf[t] = *reinterpret_cast<const uint4*>(&cs.Q[img_off<FD>(16 * t + l16, 32 * s + 4 * lq)]);
                }
            };
            load_kq(0, KF[0], QF[0]);
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int b = s & 1;
                if (s + 1 < NKS) load_kq(s + 1, KF[b ^ 1], QF[b ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        X[t][hh] = mfma_f16(KF[b][t], BS[hh][s], X[t][hh]);
                        Y[t][hh] = mfma_f16(BS[hh][s], QF[b][t], Y[t][hh]);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // R = V - e^gamma X, Delta = Mmat R, O^T = e^gamma S Q^T + Delta^T P^T
        auto step_a2 = [&](const FSlot& cs, const FV& cv, long jc) __attribute__((always_inline)) {
            const int ln = opaque(lane), l16 = ln & 15, lq = ln >> 4;
            uint4 MF[4][2], PF[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    MF[t][hf] = *reinterpret_cast<const uint4*>(&cs.M[img_off<64>(16 * t + l16, 32 * hf + 4 * lq)]);
                    PF[t][hf] = *reinterpret_cast<const uint4*>(&cs.P[img_off<64>(16 * t + l16, 32 * hf + 4 * lq)]);
                }
            // rows 16t + 4lq + v; the lane's two adjacent columns in one read
            f32x4_t R[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float4 eg = *reinterpret_cast<const float4*>(&cs.eg[16 * t + 4 * lq]);
                const float egv[4] = {eg.x, eg.y, eg.z, eg.w};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t vv = *reinterpret_cast<const uint32_t*>(&cv.v[(16 * t + 4 * lq + v) * FD + 32 * w + 2 * l16]);
                    R[t][0][v] = __uint_as_float(vv << 16) - egv[v] * X[t][0][v];
                    R[t][1][v] = __uint_as_float(vv & 0xffff0000u) - egv[v] * X[t][1][v];
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint4 BR0 = pack_f16_frag(R[0][hh], R[1][hh]), BR1 = pack_f16_frag(R[2][hh], R[3][hh]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    Dl[t][hh] = mfma_f16(MF[t][1], BR1, mfma_f16(MF[t][0], BR0, f32x4_t{0.f, 0.f, 0.f, 0.f}));
            }
            // O^T (lane: token 16t + l16, columns 32w + 8lq + 0..7), stored through a resource that
            // ends at the chunk's last token row
            f32x4_t O[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float egt = cs.eg[16 * t + l16];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) O[t][hh] = Y[t][hh] * egt;
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint4 BD0 = pack_f16_frag(Dl[0][hh], Dl[1][hh]), BD1 = pack_f16_frag(Dl[2][hh], Dl[3][hh]);
#pragma unroll
                for (int t = 0; t < 4; ++t) O[t][hh] = mfma_f16(BD1, PF[t][1], mfma_f16(BD0, PF[t][0], O[t][hh]));
            }
            if (p.o) {
                constexpr int E = (int)sizeof(TO);
                const long obos = sbos + jc * kChunk;
                const auto orr = make_rsrc(static_cast<TO*>(p.o) + (obos * H + h) * FD + 32 * w,
                                           (unsigned)(((chunk_len(jc) - 1) * H * FD + 32) * E));
#pragma unroll
                for (int t = 0; t < 4; ++t) buf_store8<TO>(orr, ((16 * t + l16) * H * FD + 8 * lq) * E, O[t][0], O[t][1]);
            }
        };

        // S^T <- e^{gamma_last} S^T + K^T diag(e^{gamma_last - gamma}) Delta
        auto step_c = [&](const FSlot& cs) __attribute__((always_inline)) {
            const int ln = opaque(lane), lq = ln >> 4, l16 = ln & 15;
            uint4 BT[2][2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x4_t Dd[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float4 ed = *reinterpret_cast<const float4*>(&cs.ed[16 * t + 4 * lq]);
                    Dd[t] = f32x4_t{ed.x * Dl[t][hh][0], ed.y * Dl[t][hh][1], ed.z * Dl[t][hh][2], ed.w * Dl[t][hh][3]};
                }
                BT[hh][0] = pack_f16_frag(Dd[0], Dd[1]);
                BT[hh][1] = pack_f16_frag(Dd[2], Dd[3]);
            }
            const float elast = cs.eg[63];
            const int tr = l16 >> 2, tc = 4 * (l16 & 3);
#pragma unroll
            for (int j = 0; j < NKB; ++j) {
                const int c = 16 * j + tc;
                const uint4 K0 = lds_frag2_t(&cs.K[img_off<FD>(4 * lq + tr, c)], &cs.K[img_off<FD>(16 + 4 * lq + tr, c)]);
                const uint4 K1 = lds_frag2_t(&cs.K[img_off<FD>(32 + 4 * lq + tr, c)], &cs.K[img_off<FD>(48 + 4 * lq + tr, c)]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    ST[hh][j] = mfma_f16(K1, BT[hh][1], mfma_f16(K0, BT[hh][0], ST[hh][j] * elast));
            }
        };

        // runs chunks c0 .. of the range and returns how many it stepped (fewer than len: it
        // stopped at a matching record, SEG >= 2)
        auto run = [&](long c0, long len, int g) __attribute__((always_inline)) -> int {
            if (len == 0) return 0;
            lds_barrier_lgkm();   // chunk c0's images written
            step_a1(slot[0]);
            lds_barrier_lgkm();
            for (int i = 0;; ++i) {
                lds_barrier_lgkm();   // B0
                if (range_done(i, len)) return i;
                step_a2(slot[i & 1], vb[i & 1], c0 + i);
                lds_barrier_lgkm();   // B1: chunk i+1's images written
                step_c(slot[i & 1]);
                const int off = i + 1;
                if constexpr (SEG == 1) {   // the walk never compares in segment 0
                    if (g > 0 && recorded(off, len)) store_state(seg_state(g, 31 - __builtin_clz(off)));
                }
                if constexpr (CMP) {
                    bool same = false;
                    if (recorded(off, len)) {
                        const float* rec = seg_state(g, 31 - __builtin_clz(off));
                        const int ln = opaque(lane);
                        unsigned diff = 0;
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                            for (int j = 0; j < NKB; ++j) {
                                const uint4 r = *reinterpret_cast<const uint4*>(rec + scol(hh, ln) + 16 * j);
                                diff |= (r.x ^ __float_as_uint(ST[hh][j][0])) | (r.y ^ __float_as_uint(ST[hh][j][1])) |
                                        (r.z ^ __float_as_uint(ST[hh][j][2])) | (r.w ^ __float_as_uint(ST[hh][j][3]));
                            }
                        same = __builtin_amdgcn_ballot_w64(diff != 0) == 0;
                    }
                    if (lane == 0) match[i & 1][w] = same ? 1 : 0;
                }
                if (i + 1 < len) step_a1(slot[(i + 1) & 1]);
                lds_barrier_lgkm();   // B2
            }
        };

        if constexpr (SEG == 3) {
            // segments 1 .. g-1 were fixed by the second pass. ok: the state SEG = 2 started the
            // current segment from was the true one; otherwise ST holds the true state entering it
            int g = walk_first_stop(reran, p.seg_n, [&](int gg) { long c0, len; seg_range(gg, c0, len); return len; });
            bool ok = true;
            int glast = g - 1;
            long c0, len;
            if (g < p.seg_n && (seg_range(g, c0, len), len > 0)) {
                glast = g;
                ok = false;
                load_state(seg_state(g, p.seg_ncp + 1));   // no match: SEG = 2's final state is the true one
                for (++g; g < p.seg_n; ++g) {
                    seg_range(g, c0, len);
                    if (len == 0) break;
                    glast = g;
                    if (ok) {
                        ok = reran[g] < len;
                        if (!ok) load_state(seg_state(g, p.seg_ncp + 1));
                        continue;
                    }
                    ok = run(c0, len, g) < len;   // matched: the true final state is SEG = 1's
                }
            }
            if (ok) load_state(seg_state(glast, p.seg_ncp));
        } else {
            const int m = run(c_first, c_count, seg);
            if constexpr (SEG == 2) {
                if (m == c_count) store_state(seg_state(seg, p.seg_ncp + 1));
                if (w == 0 && lane < FD / 64) reran[lane * p.seg_n + seg] = m;
            }
        }
        if constexpr (SEG == 1) {
            store_state(seg_state(seg, p.seg_ncp));
        } else if (SEG != 2 && p.hT) {
            store_state(p.hT + pair * FD * FD);
        }
    } else {
        // --------------------------------------------------------------- operator waves
        // one instance per operator wave index, so that every block index is a constant
        auto role = [&](auto uc) __attribute__((always_inline)) {
            constexpr int U = decltype(uc)::value;
            ORaw raw;
            auto load_raw = [&](long jc) __attribute__((always_inline)) {
                oraw_load<U>(raw, p, sbos + jc * kChunk, chunk_len(jc), h, opaque(lane));
            };
            // builds the operators of chunks c0 .., chunk c0 + j in slot[j % 2] and vb[j % 2], one
            // chunk ahead of the state waves; returns where the state waves stopped. The raw rows
            // of chunk j + 1 are loaded at the start of chunk j's phase A2 and land meanwhile.
            auto run = [&](long c0, long len) __attribute__((always_inline)) -> int {
                if (len == 0) return 0;
                load_raw(c0);
                op_a1<U>(slot[0], vb[0], ops, raw, opaque(lane));
                lds_barrier_lgkm();
                if (len > 1) load_raw(c0 + 1);
                op_a2<U>(slot[0], ops, opaque(lane));
                lds_barrier_lgkm();
                op_c<U>(slot[0], ops, opaque(lane));
                for (int i = 0;; ++i) {
                    lds_barrier_lgkm();   // B0
                    if (range_done(i, len)) return i;
                    const bool more = i + 1 < len;
                    if (more) op_a1<U>(slot[(i + 1) & 1], vb[(i + 1) & 1], ops, raw, opaque(lane));
                    lds_barrier_lgkm();   // B1
                    if (i + 2 < len) load_raw(c0 + i + 2);
                    if (more) op_a2<U>(slot[(i + 1) & 1], ops, opaque(lane));
                    lds_barrier_lgkm();   // B2
                    if (more) op_c<U>(slot[(i + 1) & 1], ops, opaque(lane));
                }
            };
            if constexpr (SEG == 3) {
                int g = walk_first_stop(reran, p.seg_n, [&](int gg) { long c0, len; seg_range(gg, c0, len); return len; });
                long c0, len;
                if (g < p.seg_n && (seg_range(g, c0, len), len > 0)) {
                    bool ok = false;
                    for (++g; g < p.seg_n; ++g) {
                        seg_range(g, c0, len);
                        if (len == 0) break;
                        if (ok) {
                            ok = reran[g] < len;
                            continue;
                        }
                        ok = run(c0, len) < len;
                    }
                }
            } else {
                run(c_first, c_count);
            }
        };
        switch (wave - NSW) {
            case 0: role(std::integral_constant<int, 0>{}); break;
            case 1: role(std::integral_constant<int, 1>{}); break;
            case 2: role(std::integral_constant<int, 2>{}); break;
            default: role(std::integral_constant<int, 3>{}); break;
        }
    }
}

// The one-kernel path holds one work-group per (sequence, head), or per segment of one, on a
// compute unit and takes about 5.5 us per chunk (the operator waves' chain of Gram blocks,
// triangular solve and products); the two-stage path spreads the operators over the whole device
// and steps the state faster. On MI355X the one-kernel path is ahead for long chains of few
// pairs (B1 H16 T32768: 0.28 against 0.35 ms) and behind from 64 pairs on (B4 H16 T2048: 0.10
// against 0.09 ms; 256 packed sequence-heads: 0.66 against 0.63 ms).
constexpr long kFusedMaxPairs = 64;

bool fused_wanted(int N, int H, int dk, int dv, int bf16) {
    if (!bf16 || dk != FD || dv != FD) return false;
    if (const char* env = std::getenv("GDN_FUSED")) return std::atoi(env) != 0;
    return (long)N * H < kFusedMaxPairs;
}

// one pass, or the three passes of the long-chain split

template <typename TO>
static hipError_t fused_launch(const ChunkProblem& p, hipStream_t s) {
    const long pairs = (long)p.N * p.H;
    const dim3 block(FNT);
    if (p.seg_n <= 1) return launch(chunk_fused_kernel<TO, 0>, dim3((unsigned)pairs), block, s, p);
    hipError_t e = launch(chunk_fused_kernel<TO, 1>, dim3((unsigned)(pairs * p.seg_n)), block, s, p);
    if (e == hipSuccess) e = launch(chunk_fused_kernel<TO, 2>, dim3((unsigned)(pairs * (p.seg_n - 1))), block, s, p);
    return e != hipSuccess ? e : launch(chunk_fused_kernel<TO, 3>, dim3((unsigned)pairs), block, s, p);
}

hipError_t launch_chunk_fused(const ChunkProblem& p, hipStream_t s) {
    if ((long)p.N * p.H == 0) return hipSuccess;
    return p.o_bf16 ? fused_launch<uint16_t>(p, s) : fused_launch<float>(p, s);
}

}  // namespace gdn
