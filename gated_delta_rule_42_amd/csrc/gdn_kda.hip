// Chunkwise forward pass of the gated delta rule with a channel-wise decay (one decay per key
// channel) for gfx950.
//
// The pages extend the gated delta rule "with a channel-wise forgetting gate" (record "LIT-137",
// "Standing in the anthology"; practice "SOTA-135", "Sequence": it "replaces the scalar decay
// with a channel-wise one") and give no formula. Reading: alpha_t becomes a vector in
// (0,1]^{d_k} applied to the key channels (the columns of S [d_v, d_k]) where the scalar one
// was, before the write:
//     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
// Chunk form (derived; the scalar case with the row scalings of K and Q replaced by
// elementwise ones): with gamma_r the in-chunk cumulative log decay of every channel,
// Kh = K * e^gamma, Qh = Q * e^gamma, Kd = K * e^{gamma_last - gamma}, lam = e^{gamma_last}:
//     A     = strict_lower(diag(beta) [sum_c k_r k_i e^{gamma_r - gamma_i}])
//     T     = (I + A)^{-1},   Mmat = T diag(beta)
//     P     = lower_incl([sum_c q_r k_i e^{gamma_r - gamma_i}])
//     Delta = Mmat (V - Kh S^T),   O = Qh S^T + P Delta,   S' = S Diag(lam) + Delta^T Kd.
// With decoupled erase and write gates (record "LIT-137", "Standing in the anthology": beta
// split into a channel-wise erase gate on the key and a channel-wise write gate on the value;
// practice "SOTA-135": the erased read runs along a reweighted key) the erased read runs along
// E * k and the written value is W * v: the same chunk form with A's left factor E * K instead
// of diag(beta) K, Kh = E * K * e^gamma, V replaced by W * V and Mmat = T.
// Stage 1 (kda_prepare_kernel) forms Kh, Qh, Kd, lam, Mmat and P per (chunk, head) in fp32 (bf16
// inputs widened on load; the operators are stored as fp16 for bf16 inputs; for bf16 inputs the
// Gram blocks below the diagonal blocks take fp16 operands and the diagonal blocks bf16 hi + lo
// pairs, see gram_rows_of); stage 2 carries the
// fp32 state through the chunks: kda_propagate_kernel for fp32 inputs (fp32 16x16x4 matrix core),
// for bf16 inputs kda_propagate_dma_kernel (operators copied into LDS by a DMA wave from the
// images stage 1 writes; with decoupled gates the write gate is copied beside V), on the fp16
// 16x16x32 matrix core with fp32 accumulation.
//
// A and P never form e^{-gamma} (it overflows under strong decay): every 16-row block uses a
// reference at its first row, so the factor e^{gamma_r - gamma_ref} of a row is <= 1 and
// e^{gamma_ref - gamma_i} of a column is <= 1 below the diagonal block and at most
// e^kMaxRange within it; channels that decay more than that over a block are summed exactly
// there, term by term.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_stage2.h"
#include "gdn_ut.h"

#include <type_traits>

namespace gdn {

// Four consecutive input elements as fp32.
__device__ __forceinline__ float4 load4_in(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_in(const uint16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// Four fp32 values stored as the operand type (fp32, or fp16 for bf16 inputs).
__device__ __forceinline__ void put4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ void put4(_Float16* p, float4 x) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_f16x2(x.x, x.y), pack_f16x2(x.z, x.w));
}

// ------------------------------------------------------------------- stage 1
template <int DK>
struct alignas(16) KdaPrepSmem {
    static constexpr int PK = DK + 4, PF = 68;
    float K[64 * PK];
    float Q[64 * PK];
    float G[64 * PK];   // g, then gamma (in-chunk inclusive cumulative sum, per channel)
    float A[64 * PF];
    float T[64 * PF];   // before the Gram products: per row block of the gamma scan, the
                        // block's sum of g per channel; during them, their scratch
    float P[64 * PF];   // with decoupled gates, until A is formed: the raw Q tile
    float beta[64];
};

// Threads of the stage-1 work-group: eight waves, two per SIMD, so that one wave's LDS and
// transcendental latencies hide behind the other's work.
constexpr int kKdaPrepThreads = 512;

// Rows of row block I of [sum_c L[r][c] K[i][c] e^{gamma_r[c] - gamma_i[c]}], i < 16 (I + 1),
// for one or two left operands L1, L2 (sharing the right operand K and the exponentials), into
// O1 (times rs1[r] when rs1 is set; strictly lower when strict1) and O2 (lower including the
// diagonal). Two waves share a row block, each summing half of the d_k channels (HF = 0: the
// first half); the first writes its partial sums, the second adds its own after a barrier.
// Column blocks on the fp32 matrix core with the reference gamma of row 16 I:
// left factor L[r] e^{gamma_r - gamma_ref} (<= |L|: r >= ref), right factor
// K[i] e^{gamma_ref - gamma_i}, which is <= |K| below the diagonal block (i < ref) and, in the
// diagonal block, grows with the channel's decay over the block's rows. A channel whose decay
// over the block exceeds e^kMaxRange is left out of the diagonal block's product and summed
// there exactly instead (one exponent per term), so no factor exceeds e^kMaxRange.
//
// F16 (bf16 inputs): the blocks below the diagonal block (J < I) go to the fp16 matrix core
// instead, factored through the last row of column block J: the left factor
// L[r] e^{gamma_r - gamma_last(J)} = (L[r] e^{gamma_r - gamma_ref}) e^{gamma_ref - gamma_last(J)}
// and the right factor K[i] e^{gamma_last(J) - gamma_i} are both <= |L|, |K| (rows r > last(J)
// >= i, and gamma does not increase down the chunk), so nothing overflows fp16; a factor that
// underflows belongs to a term below fp16's resolution of the entry. The right factors depend
// on J alone: the waves of row block J form them once as fp16 fragments (zf) for the waves
// below, and those of row block I form its channel scalars e^{gamma_ref - gamma_last(J)} (ss);
// see gram_offdiag_prep. The
// diagonal block (F16) runs on the bf16 matrix core with each factor as a bf16 hi + lo pair.
constexpr float kMaxRange = 60.f;

// Scratch of the fp16 off-diagonal products (in the T buffer, which the UT transform fills
// only after the Gram products): zf[J][s][lane] = the right-operand fragment of column block J
// (J < 3) for d_k slice s, ss[pair][c] = e^{gamma_ref(I) - gamma_last(J)} for pair
// I (I - 1) / 2 + J.
template <int DK>
struct KdaOffdiag {
    static constexpr int NS = DK / 32;
    static constexpr int BYTES = 3 * NS * 64 * 16 + 6 * DK * 4;
    uint4* zf;
    float* ss;
    __device__ __forceinline__ explicit KdaOffdiag(float* base)
        : zf(reinterpret_cast<uint4*>(base)), ss(base + 3 * NS * 64 * 4) {}
};

// A wave's share of the scratch of row block I, the channel half HF of: the right-operand
// fragments of column block I (I < 3; lane (l16, lq) holds row 16 I + l16, channels
// 32 s + 4 lq + 0..3 and 32 s + 16 + 4 lq + 0..3, the k-slot order of the products) and the
// channel scalars of its pairs (I > 0).
template <int DK, int I, int HF>
__device__ __forceinline__ void gram_offdiag_prep(const KdaPrepSmem<DK>& sm, KdaOffdiag<DK> od, int lane) {
    constexpr int PK = KdaPrepSmem<DK>::PK, NS = KdaOffdiag<DK>::NS;
    const int l16 = lane & 15, lq = lane >> 4;
    if constexpr (I < 3) {
        const int i = 16 * I + l16, last = 16 * I + 15;
#pragma unroll
        for (int s = HF * NS / 2; s < (HF + 1) * NS / 2; ++s) {
            const int c0 = 32 * s + 4 * lq;
            uint32_t w[4];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4_t k = *reinterpret_cast<const f32x4_t*>(&sm.K[i * PK + c0 + 16 * hf]);
                const f32x4_t g = *reinterpret_cast<const f32x4_t*>(&sm.G[i * PK + c0 + 16 * hf]);
                const f32x4_t gl = *reinterpret_cast<const f32x4_t*>(&sm.G[last * PK + c0 + 16 * hf]);
                w[2 * hf] = pack_f16x2(k[0] * __expf(gl[0] - g[0]), k[1] * __expf(gl[1] - g[1]));
                w[2 * hf + 1] = pack_f16x2(k[2] * __expf(gl[2] - g[2]), k[3] * __expf(gl[3] - g[3]));
            }
            od.zf[(I * NS + s) * 64 + lane] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
#pragma unroll
    for (int J = 0; J < I; ++J)
#pragma unroll
        for (int c0 = 64 * HF; c0 < DK; c0 += 128) {
            const int c = c0 + lane;
            od.ss[(I * (I - 1) / 2 + J) * DK + c] = __expf(sm.G[16 * I * PK + c] - sm.G[(16 * J + 15) * PK + c]);
        }
}

template <int DK, bool TWO, int I, bool F16, int HF>
__device__ __forceinline__ void gram_rows_of(const KdaPrepSmem<DK>& sm, const float* L1, const float* L2,
                                             float* O1, float* O2, const float* rs1, bool strict1,
                                             KdaOffdiag<DK> od, int lane) {
    constexpr int PK = KdaPrepSmem<DK>::PK, PF = KdaPrepSmem<DK>::PF;
    const int l16 = lane & 15, lq = lane >> 4;
    f32x4_t a1[4], a2[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) a1[J] = a2[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (F16) {
        // One pass per 32-channel slice over the lane's row r = 16 I + l16 (channels
        // 32 s + 4 lq + 0..3 and the same + 16): the left factors L e^{gamma_r - gamma_ref}
        // serve both products.
        // Below the diagonal block (J < I): fp16 operands, the left factor times the channel
        // scalars e^{gamma_ref - gamma_last(J)} against wave J's right-factor fragments.
        // The diagonal block on the bf16 matrix core (16x16x32): bf16 keeps fp32's exponent
        // range, so the factors up to e^kMaxRange fit; each factor is a bf16 hi + lo pair and a
        // slice takes three products (hi hi, hi lo, lo hi), about 16 significant bits per
        // factor; the lane gives row r both as the left operand and as the right one.
        constexpr int NS = KdaOffdiag<DK>::NS;
        const int r = 16 * I + l16;
#pragma unroll 1
        for (int s = HF * NS / 2; s < (HF + 1) * NS / 2; ++s) {
            const int c0 = 32 * s + 4 * lq;
            f32x4_t x1[2], x2[2], y[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int c = c0 + 16 * hf;
                const f32x4_t g = *reinterpret_cast<const f32x4_t*>(&sm.G[r * PK + c]);
                const f32x4_t gf = *reinterpret_cast<const f32x4_t*>(&sm.G[16 * I * PK + c]);
                const f32x4_t gl = *reinterpret_cast<const f32x4_t*>(&sm.G[(16 * I + 15) * PK + c]);
                const f32x4_t k = *reinterpret_cast<const f32x4_t*>(&sm.K[r * PK + c]);
                const f32x4_t l1 = *reinterpret_cast<const f32x4_t*>(&L1[r * PK + c]);
                f32x4_t l2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if constexpr (TWO) l2 = *reinterpret_cast<const f32x4_t*>(&L2[r * PK + c]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float el = __expf(g[e] - gf[e]);
                    x1[hf][e] = l1[e] * el;
                    x2[hf][e] = l2[e] * el;
                    y[hf][e] = gf[e] - gl[e] <= kMaxRange ? k[e] * __expf(gf[e] - g[e]) : 0.f;
                }
            }
#pragma unroll
            for (int J = 0; J < I; ++J) {
                const float* sc = od.ss + (I * (I - 1) / 2 + J) * DK;
                const f32x4_t sa = *reinterpret_cast<const f32x4_t*>(&sc[c0]);
                const f32x4_t sb = *reinterpret_cast<const f32x4_t*>(&sc[c0 + 16]);
                const uint4 bz = od.zf[(J * NS + s) * 64 + lane];
                const uint4 f1 = make_uint4(pack_f16x2(x1[0][0] * sa[0], x1[0][1] * sa[1]), pack_f16x2(x1[0][2] * sa[2], x1[0][3] * sa[3]),
                                            pack_f16x2(x1[1][0] * sb[0], x1[1][1] * sb[1]), pack_f16x2(x1[1][2] * sb[2], x1[1][3] * sb[3]));
                a1[J] = mfma_f16(f1, bz, a1[J]);
                if constexpr (TWO) {
                    const uint4 f2 = make_uint4(pack_f16x2(x2[0][0] * sa[0], x2[0][1] * sa[1]), pack_f16x2(x2[0][2] * sa[2], x2[0][3] * sa[3]),
                                                pack_f16x2(x2[1][0] * sb[0], x2[1][1] * sb[1]), pack_f16x2(x2[1][2] * sb[2], x2[1][3] * sb[3]));
                    a2[J] = mfma_f16(f2, bz, a2[J]);
                }
            }
            uint4 yh, yl, xh, xl;
            split_bf16_frag(y[0], y[1], yh, yl);
            split_bf16_frag(x1[0], x1[1], xh, xl);
            a1[I] = mfma_bf16(xh, yh, a1[I]);
            a1[I] = mfma_bf16(xh, yl, a1[I]);
            a1[I] = mfma_bf16(xl, yh, a1[I]);
            if constexpr (TWO) {
                split_bf16_frag(x2[0], x2[1], xh, xl);
                a2[I] = mfma_bf16(xh, yh, a2[I]);
                a2[I] = mfma_bf16(xh, yl, a2[I]);
                a2[I] = mfma_bf16(xl, yh, a2[I]);
            }
        }
    } else {
        // fp32 products: lane (l16, lq) takes channels 16 u + 4 lq + e, e = 0..3, in product (u, e),
        // so its operands arrive as 16-byte reads
        constexpr int J0 = 0;
        for (int u = HF * DK / 32; u < (HF + 1) * DK / 32; ++u) {
            const int c = 16 * u + 4 * lq;
            const f32x4_t gref = *reinterpret_cast<const f32x4_t*>(&sm.G[16 * I * PK + c]);
            const f32x4_t glast = *reinterpret_cast<const f32x4_t*>(&sm.G[(16 * I + 15) * PK + c]);
            const f32x4_t grow = *reinterpret_cast<const f32x4_t*>(&sm.G[(16 * I + l16) * PK + c]);
            const f32x4_t l1 = *reinterpret_cast<const f32x4_t*>(&L1[(16 * I + l16) * PK + c]);
            f32x4_t l2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (TWO) l2 = *reinterpret_cast<const f32x4_t*>(&L2[(16 * I + l16) * PK + c]);
            f32x4_t kj[I + 1], gj[I + 1];
    #pragma unroll
            for (int J = J0; J <= I; ++J) {
                kj[J] = *reinterpret_cast<const f32x4_t*>(&sm.K[(16 * J + l16) * PK + c]);
                gj[J] = *reinterpret_cast<const f32x4_t*>(&sm.G[(16 * J + l16) * PK + c]);
            }
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool fits = gref[e] - glast[e] <= kMaxRange;
                const float el = __expf(grow[e] - gref[e]);
                const float x1 = l1[e] * el, x2 = l2[e] * el;
    #pragma unroll
                for (int J = J0; J <= I; ++J) {
                    const float b = kj[J][e] * __expf(gref[e] - gj[J][e]);
                    const float bb = (J < I || fits) ? b : 0.f;
                    a1[J] = mfma4(x1, bb, a1[J]);
                    if constexpr (TWO) a2[J] = mfma4(x2, bb, a2[J]);
                }
            }
        }
    }
    if constexpr (HF == 0) {
#pragma unroll
        for (int J = 0; J <= I; ++J) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * I + 4 * lq + m, i = 16 * J + l16;
                const bool k1 = J < I || (strict1 ? i < r : i <= r), k2 = J < I || i <= r;
                O1[r * PF + i] = k1 ? (rs1 ? rs1[r] : 1.f) * a1[J][m] : 0.f;
                if constexpr (TWO) O2[r * PF + i] = k2 ? a2[J][m] : 0.f;
            }
        }
    }
    __syncthreads();  // the first half's sums are in O1, O2
    if constexpr (HF == 0) return;
#pragma unroll
    for (int J = 0; J <= I; ++J) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * I + 4 * lq + m, i = 16 * J + l16;
            const bool k1 = J < I || (strict1 ? i < r : i <= r), k2 = J < I || i <= r;
            if (k1) O1[r * PF + i] += (rs1 ? rs1[r] : 1.f) * a1[J][m];
            if constexpr (TWO)
                if (k2) O2[r * PF + i] += a2[J][m];
        }
    }
    // channels left out of the diagonal block's product: exact sums over them (each lane adds to
    // the entries it added to above)
    for (int c0 = 0; c0 < DK; c0 += 64) {
        const int ch = c0 + lane;
        const bool out = ch < DK && sm.G[16 * I * PK + ch] - sm.G[(16 * I + 15) * PK + ch] > kMaxRange;
        unsigned long long bits = __ballot(out);
        while (bits) {
            const int c = c0 + __builtin_ctzll(bits);
            bits &= bits - 1;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * I + 4 * lq + m, i = 16 * I + l16;
                if (i <= r) {
                    const float e = __expf(sm.G[r * PK + c] - sm.G[i * PK + c]) * sm.K[i * PK + c];
                    if (strict1 ? i < r : true) O1[r * PF + i] += (rs1 ? rs1[r] : 1.f) * L1[r * PK + c] * e;
                    if constexpr (TWO) O2[r * PF + i] += L2[r * PK + c] * e;
                }
            }
        }
    }
}

// gram_rows_of for the (row block, channel half) of this wave; both are compile-time constants
// of each wave's code, so its loops are static. Wave w and w + 4 share a SIMD; the pairing puts
// the longest and the shortest row block (3 and 0), or 2 and 1, on each SIMD, so that every SIMD
// gets the same work: waves 0-3 take row blocks 3, 3, 2, 2 and waves 4-7 row blocks 0, 0, 1, 1,
// halves alternating. (F16: the scratch is filled first, then a barrier.) Called by all
// kKdaPrepThreads threads; takes two barriers (one without F16).
template <int DK, bool TWO, bool F16>
__device__ __forceinline__ void gram_rows(const KdaPrepSmem<DK>& sm, const float* L1, const float* L2,
                                          float* O1, float* O2, const float* rs1, bool strict1,
                                          float* scratch, int wave, int lane) {
    const KdaOffdiag<DK> od(scratch);
    auto run = [&](auto ib, auto hf) {
        constexpr int I = decltype(ib)::value, HF = decltype(hf)::value;
        if constexpr (F16) {
            gram_offdiag_prep<DK, I, HF>(sm, od, lane);
            __syncthreads();
        }
        gram_rows_of<DK, TWO, I, F16, HF>(sm, L1, L2, O1, O2, rs1, strict1, od, lane);
    };
    using std::integral_constant;
    switch (wave) {
        case 0: run(integral_constant<int, 3>{}, integral_constant<int, 0>{}); break;
        case 1: run(integral_constant<int, 3>{}, integral_constant<int, 1>{}); break;
        case 2: run(integral_constant<int, 2>{}, integral_constant<int, 0>{}); break;
        case 3: run(integral_constant<int, 2>{}, integral_constant<int, 1>{}); break;
        case 4: run(integral_constant<int, 0>{}, integral_constant<int, 0>{}); break;
        case 5: run(integral_constant<int, 0>{}, integral_constant<int, 1>{}); break;
        case 6: run(integral_constant<int, 1>{}, integral_constant<int, 0>{}); break;
        default: run(integral_constant<int, 1>{}, integral_constant<int, 1>{}); break;
    }
}

// One (chunk, head) unit's stage-1 inputs, staged in registers: K, g and Q (or, with decoupled
// gates, the erase gate), 4 values per group, and beta. Every load is issued unconditionally,
// rows past the chunk's end through buffer resources that read them as zeros; the element
// arrays use native vector types (a struct-typed copy would go through memory).
template <typename TIn, int DK, bool DEC>
struct KdaPrepStage {
    static constexpr int NP = 64 * DK / 4 / kKdaPrepThreads;   // groups of 4 values per thread
    // thread tid holds channels 4 (tid % NG) .. +3 of the NP consecutive rows NP (tid / NG) + it
    static constexpr int NG = DK / 4, RB = kKdaPrepThreads / NG;
    static constexpr int EB = (int)sizeof(TIn);    // bytes of an input element
    // with decoupled gates Q is staged too when its raw tile fits in the P buffer (all shapes
    // but fp32 d_k = 128, which loads it when needed)
    static constexpr bool QPRE = !DEC || 64 * DK * EB <= (int)sizeof(KdaPrepSmem<DK>::P);
    static_assert(RB * DK <= (int)sizeof(KdaPrepSmem<DK>::T) / 4, "the scan's block sums fit in T");
    u32x4_t k[NP], q[NP];                         // raw groups (bf16: the low 8 bytes)
    f32x4_t g[NP], e[NP];
    float beta;

    __device__ __forceinline__ static u32x4_t raw4(__amdgpu_buffer_rsrc_t r, int off) {
        if constexpr (EB == 2) {
            const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            return u32x4_t{x[0], x[1], 0u, 0u};
        } else {
            return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        }
    }
    __device__ __forceinline__ static float4 widen(u32x4_t x) {
        if constexpr (EB == 2)
            return make_float4(__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u),
                               __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xffff0000u));
        else
            return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
    }

    __device__ __forceinline__ void load(const ChunkProblem& p, long bos, int len, int h, int tid) {
        const int H = p.H;
        const long o = (bos * H + h) * DK;
        const unsigned rows = (unsigned)((len - 1) * H * DK + DK);
        const auto kr = make_rsrc(static_cast<const TIn*>(p.k) + o, rows * EB);
        const auto qr = make_rsrc(static_cast<const TIn*>(p.q) + o, QPRE ? rows * EB : 0u);
        const auto gr = make_rsrc(p.g + o, rows * 4);
        const auto er = make_rsrc(DEC ? p.erase + o : p.g, DEC ? rows * 4 : 0u);
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int r = NP * (tid / NG) + it, cc = 4 * (tid % NG), x = r * H * DK + cc;
            k[it] = raw4(kr, x * EB);
            q[it] = raw4(qr, x * EB);
            g[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(gr, x * 4, 0, 0));
            e[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(er, x * 4, 0, 0));
        }
        const auto br = make_rsrc(p.beta + bos * H + h, DEC ? 0u : (unsigned)(((len - 1) * H + 1) * 4));
        beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(br, tid * H * 4, 0, 0));
    }

    // K and (Q, or E * K with decoupled gates) into LDS as fp32, and with decoupled gates the raw
    // Q tile into P ([64, DK] row-major input elements); g scanned down the thread's rows in
    // registers, the row block's sum into T
    __device__ __forceinline__ void store(KdaPrepSmem<DK>& sm, int tid) {
        constexpr int PK = KdaPrepSmem<DK>::PK;
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int r = NP * (tid / NG) + it, cc = 4 * (tid % NG);
            const float4 kv = widen(k[it]);
            const float4 qv = DEC ? make_float4(e[it][0] * kv.x, e[it][1] * kv.y, e[it][2] * kv.z, e[it][3] * kv.w)
                                  : widen(q[it]);
            *reinterpret_cast<float4*>(&sm.K[r * PK + cc]) = kv;
            *reinterpret_cast<float4*>(&sm.Q[r * PK + cc]) = qv;
            if constexpr (DEC && QPRE) {
                char* dst = reinterpret_cast<char*>(sm.P) + (r * DK + cc) * EB;
                if constexpr (EB == 2) *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{q[it][0], q[it][1]};
                else *reinterpret_cast<u32x4_t*>(dst) = q[it];
            }
            if (it > 0) g[it] += g[it - 1];
        }
        *reinterpret_cast<f32x4_t*>(&sm.T[(tid / NG) * DK + 4 * (tid % NG)]) = g[NP - 1];
        if (tid < 64) sm.beta[tid] = beta;
    }
    // with decoupled gates: the raw Q tile in P to fp32 in Q (rows past the chunk's end are zero,
    // as loaded)
    __device__ __forceinline__ static void q_from_raw(KdaPrepSmem<DK>& sm, int tid) {
        constexpr int PK = KdaPrepSmem<DK>::PK;
        for (int i = tid; i < 64 * DK / 4; i += kKdaPrepThreads) {
            const int r = i / (DK / 4), cc = 4 * (i % (DK / 4));
            const char* src = reinterpret_cast<const char*>(sm.P) + (r * DK + cc) * EB;
            u32x4_t x;
            if constexpr (EB == 2) {
                const u32x2_t h = *reinterpret_cast<const u32x2_t*>(src);
                x = u32x4_t{h[0], h[1], 0u, 0u};
            } else {
                x = *reinterpret_cast<const u32x4_t*>(src);
            }
            *reinterpret_cast<float4*>(&sm.Q[r * PK + cc]) = widen(x);
        }
    }
    // gamma (the in-chunk inclusive cumulative sum of g, per channel) into LDS: the thread's
    // rows plus the sums of the row blocks above them; and the scaled operators of those rows
    // straight from registers: Kh (E * K * e^gamma with decoupled gates), Qh (not with
    // decoupled gates, whose Q is loaded later), Kd and lam, at element offset widx * 64 * DK +
    // (IMG ? the image offset : row-major). Between a barrier after store and one before gamma
    // is read.
    template <bool IMG, typename TM>
    __device__ __forceinline__ void finish_scan(KdaPrepSmem<DK>& sm, int tid, TM* khat, TM* qhat, TM* kdec,
                                                float* lam, long widx) const {
        constexpr int PK = KdaPrepSmem<DK>::PK;
        const int rb = tid / NG, cc = 4 * (tid % NG);
        f32x4_t pre = {0.f, 0.f, 0.f, 0.f}, last = pre;   // rows above the block; gamma_last
        for (int b = 0; b < RB; ++b) {
            if (b == rb) pre = last;
            last += *reinterpret_cast<const f32x4_t*>(&sm.T[b * DK + cc]);
        }
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int r = NP * rb + it;
            const f32x4_t gm = g[it] + pre;
            *reinterpret_cast<f32x4_t*>(&sm.G[r * PK + cc]) = gm;
            const float4 kv = widen(k[it]);
            const float4 x = DEC ? make_float4(e[it][0] * kv.x, e[it][1] * kv.y, e[it][2] * kv.z, e[it][3] * kv.w)
                                 : widen(q[it]);
            const float4 eg = make_float4(__expf(gm[0]), __expf(gm[1]), __expf(gm[2]), __expf(gm[3]));
            const float4 ed = make_float4(__expf(last[0] - gm[0]), __expf(last[1] - gm[1]), __expf(last[2] - gm[2]),
                                          __expf(last[3] - gm[3]));
            const long o = widx * 64 * DK + (IMG ? img_off<DK>(r, cc) : r * DK + cc);
            const float4 xs = make_float4(x.x * eg.x, x.y * eg.y, x.z * eg.z, x.w * eg.w);
            put4(khat + o, DEC ? xs : make_float4(kv.x * eg.x, kv.y * eg.y, kv.z * eg.z, kv.w * eg.w));
            put4(kdec + o, make_float4(kv.x * ed.x, kv.y * ed.y, kv.z * ed.z, kv.w * ed.w));
            if constexpr (!DEC) put4(qhat + o, xs);
        }
        if (rb == 0)
            *reinterpret_cast<float4*>(lam + widx * DK + cc) =
                make_float4(__expf(last[0]), __expf(last[1]), __expf(last[2]), __expf(last[3]));
    }
};

// Persistent work-groups: each walks (chunk, head) units with a stride of the grid, keeping the
// next unit's inputs in flight in registers while the current one is computed (the loads are
// issued on every pass, for the current unit again past the last one, which keeps the
// compiler's waits for them exact). Two waves share each row block of A and P (gram_rows). With
// decoupled gates (DEC) the erased read runs along E * K, so A's left operand is E * K (held
// in the Q buffer until A is formed, then Q is moved there from its raw copy in P), Kh is
// E * K * e^gamma, V is scaled by the write gate in stage 2 and Mmat is T itself.
template <typename TIn, int DK, bool DEC>
__global__ __launch_bounds__(kKdaPrepThreads) void kda_prepare_kernel(ChunkProblem p) {
    using SM = KdaPrepSmem<DK>;
    constexpr int PK = SM::PK, PF = SM::PF;
    constexpr bool F16 = sizeof(TIn) == 2;  // off-diagonal Gram blocks on the fp16 matrix core
    // bf16: the operators go out as the LDS images the DMA-fed stage 2 copies
    // (kda_propagate_dma_kernel); fp32: row-major
    constexpr bool IMG = sizeof(TIn) == 2;
    static_assert(KdaOffdiag<DK>::BYTES <= (int)sizeof(SM::T), "off-diagonal scratch fits in T");
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = p.H;
    const long nunits = p.nc_bound * H;
    const TIn* qp = static_cast<const TIn*>(p.q);
    using TM = typename Operand<TIn>::type;   // operators are written as fp16 for bf16 inputs
    TM* khat = reinterpret_cast<TM*>(p.khat);
    TM* qhat = reinterpret_cast<TM*>(p.qhat);
    TM* kdec = reinterpret_cast<TM*>(p.kdec);

    KdaPrepStage<TIn, DK, DEC> stage;
    long unit = blockIdx.x, bos = 0;
    int len = 0;
    bool ok = unit < nunits && locate_chunk(p, unit / H, bos, len);
    if (ok) stage.load(p, bos, len, (int)(unit % H), tid);
    while (unit < nunits) {
        const long nxt = unit + gridDim.x;
        long nbos = 0;
        int nlen = 0;
        const bool nok = nxt < nunits && locate_chunk(p, nxt / H, nbos, nlen);
        if (!ok) {
            if (nok) stage.load(p, nbos, nlen, (int)(nxt % H), tid);
            unit = nxt; ok = nok; bos = nbos; len = nlen;
            continue;
        }
        const int h = (int)(unit % H);
        const long widx = unit;   // (chunk, head) = (unit / H, unit % H)
        // Every phase takes the thread's index through opaque(), so that the per-thread addresses
        // of one phase are formed there instead of being hoisted out of the unit loop and held
        // (or spilled) through the others.
        __syncthreads();  // the previous unit is done with LDS
        stage.store(sm, opaque(tid));
        __syncthreads();
        // gamma (rows past the chunk's end add 0) and Kh, Qh, Kd, lam to the workspace
        stage.template finish_scan<IMG>(sm, opaque(tid), khat, qhat, kdec, p.lam, widx);
        __syncthreads();
        // the next unit's loads, issued past the barrier so that no wave waits there for another
        // wave's loads to be accepted behind the stores above; the Gram products hide them
        if (nok) stage.load(p, nbos, nlen, (int)(nxt % H), opaque(tid));
        else stage.load(p, bos, len, h, opaque(tid));

        // -- Qh with decoupled gates (Q is loaded after A is formed)
        auto write_qhat = [&]() {
            for (int i = opaque(tid); i < 64 * DK / 4; i += kKdaPrepThreads) {
                const int r = i / (DK / 4), cc = 4 * (i % (DK / 4));
                const float4 g = *reinterpret_cast<const float4*>(&sm.G[r * PK + cc]);
                const float4 q = *reinterpret_cast<const float4*>(&sm.Q[r * PK + cc]);
                const long o = widx * 64 * DK + (IMG ? img_off<DK>(r, cc) : r * DK + cc);
                put4(qhat + o, make_float4(q.x * __expf(g.x), q.y * __expf(g.y), q.z * __expf(g.z), q.w * __expf(g.w)));
            }
        };

        // -- A and P
        if constexpr (DEC) {
            gram_rows<DK, false, F16>(sm, sm.Q, nullptr, sm.A, nullptr, nullptr, true, sm.T, wave, opaque(lane));
            __syncthreads();  // E * K is dead: Q in its place
            if constexpr (KdaPrepStage<TIn, DK, DEC>::QPRE) {
                KdaPrepStage<TIn, DK, DEC>::q_from_raw(sm, opaque(tid));
            } else {
                for (int i = opaque(tid); i < 64 * DK / 4; i += kKdaPrepThreads) {
                    const int r = i / (DK / 4), cc = 4 * (i % (DK / 4));
                    float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (r < len) qv = load4_in(qp + ((bos + r) * H + h) * DK + cc);
                    *reinterpret_cast<float4*>(&sm.Q[r * PK + cc]) = qv;
                }
            }
            __syncthreads();
            write_qhat();
            gram_rows<DK, false, F16>(sm, sm.Q, nullptr, sm.P, nullptr, nullptr, false, sm.T, wave, opaque(lane));
        } else {
            gram_rows<DK, true, F16>(sm, sm.K, sm.Q, sm.A, sm.P, sm.beta, true, sm.T, wave, opaque(lane));
        }
        __syncthreads();

        ut_inverse64<PF>(sm.A, sm.T, wave, opaque(lane));

        // -- Mmat = T diag(beta) (T with decoupled gates) and P (lower incl. diagonal), fp32 row-major
        {
            constexpr int NE = 64 * 64 / kKdaPrepThreads;   // entries of one row per thread
            const int t = opaque(tid), r = t / (64 / NE), c0 = (t % (64 / NE)) * NE;
            float mv[NE], pv[NE];
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int ci = c0 + e;
                mv[e] = ((ci >> 4) <= (r >> 4)) ? sm.T[r * PF + ci] * (DEC ? 1.f : sm.beta[ci]) : 0.f;
                pv[e] = ci <= r ? sm.P[r * PF + ci] : 0.f;
            }
#pragma unroll
            for (int q4 = 0; q4 < NE / 4; ++q4) {
                const int o = IMG ? img_off<64>(r, c0 + 4 * q4) : r * 64 + c0 + 4 * q4;
                put4(static_cast<TM*>(p.mmat) + widx * 4096 + o,
                     make_float4(mv[4 * q4], mv[4 * q4 + 1], mv[4 * q4 + 2], mv[4 * q4 + 3]));
                put4(static_cast<TM*>(p.pmat) + widx * 4096 + o,
                     make_float4(pv[4 * q4], pv[4 * q4 + 1], pv[4 * q4 + 2], pv[4 * q4 + 3]));
            }
        }
        unit = nxt; ok = nok; bos = nbos; len = nlen;
    }
}

// ------------------------------------------------------------------- stage 2
template <int DK, int DVT>
struct alignas(16) KdaPropSmem {
    static constexpr int PK = DK + 4, PC = 68, PV = DVT + 4;
    float Kh[64 * PK];
    float Qh[64 * PK];
    float Kd[64 * PK];
    float M[64 * PC];
    float P[64 * PC];
    float V[64 * PV];
    float lam[DK];
};

// One work-group per (sequence, head, DVT-column tile); wave w owns d_v columns dv0 + 16w ..
// +15 and holds S^T [d_k, 16] as d_k/16 accumulator tiles (lane: S[col l16][16j + 4lq + 0..3]).
template <typename TIn, typename TO, int DK, int DV, int DVT>
__global__ __launch_bounds__(DVT / 16 * 64) void kda_propagate_kernel(ChunkProblem p) {
    using SM = KdaPropSmem<DK, DVT>;
    constexpr int PK = SM::PK, PC = SM::PC, PV = SM::PV, NKB = DK / 16, NTILE = DV / DVT;
    constexpr int NT = DVT / 16 * 64;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;
    const long slot = blockIdx.x / NTILE;
    const int tile = (int)(blockIdx.x % NTILE);
    // the work-group's (sequence, head) pair: packed sequences are taken longest first (the chunk
    // table's order)
    const int n = p.cu_seqlens ? p.chunk_base[p.N + 1 + (int)(slot / H)] : (int)(slot / H);
    const int h = (int)(slot % H);
    const long pair = (long)n * H + h;
    const int dv0 = tile * DVT, dvw = dv0 + 16 * wave;

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    const long cbase = (p.cu_seqlens == nullptr) ? (long)n * p.nc_per_seq : (long)p.chunk_base[n];
    long nchunks = (seos - sbos + 63) / 64;
    if (cbase + nchunks > p.nc_bound) nchunks = max(0L, p.nc_bound - cbase);

    f32x4_t ST[NKB];
    const long srow = (pair * DV + dvw + l16) * DK + 4 * lq;
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        if (p.h0) {
            const float4 x = *reinterpret_cast<const float4*>(p.h0 + srow + 16 * j);
            ST[j] = f32x4_t{x.x, x.y, x.z, x.w};
        } else {
            ST[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    const TIn* vp = static_cast<const TIn*>(p.v);
    const float* mp = static_cast<const float*>(p.mmat);
    const float* pp = static_cast<const float*>(p.pmat);

    for (long jc = 0; jc < nchunks; ++jc) {
        const long bos = sbos + jc * 64, widx = (cbase + jc) * H + h;
        const int len = (int)min(64L, seos - bos);
        __syncthreads();  // the previous chunk's LDS data is dead
        for (int i = tid; i < 64 * DK / 4; i += NT) {
            const int r = i / (DK / 4), cc = 4 * (i % (DK / 4));
            const long o = (widx * 64 + r) * DK + cc;
            *reinterpret_cast<float4*>(&sm.Kh[r * PK + cc]) = *reinterpret_cast<const float4*>(p.khat + o);
            *reinterpret_cast<float4*>(&sm.Qh[r * PK + cc]) = *reinterpret_cast<const float4*>(p.qhat + o);
            *reinterpret_cast<float4*>(&sm.Kd[r * PK + cc]) = *reinterpret_cast<const float4*>(p.kdec + o);
        }
        for (int i = tid; i < 64 * 16; i += NT) {
            const int r = i / 16, cc = 4 * (i % 16);
            *reinterpret_cast<float4*>(&sm.M[r * PC + cc]) = *reinterpret_cast<const float4*>(mp + widx * 4096 + r * 64 + cc);
            *reinterpret_cast<float4*>(&sm.P[r * PC + cc]) = *reinterpret_cast<const float4*>(pp + widx * 4096 + r * 64 + cc);
        }
        for (int i = tid; i < 64 * DVT / 4; i += NT) {
            const int r = i / (DVT / 4), cc = 4 * (i % (DVT / 4));
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < len) {
                const long o = ((bos + r) * H + h) * DV + dv0 + cc;
                x = load4_in(vp + o);
                if (p.write) {   // decoupled gates: the written value is w * v
                    const float4 w = *reinterpret_cast<const float4*>(p.write + o);
                    x = make_float4(x.x * w.x, x.y * w.y, x.z * w.z, x.w * w.w);
                }
            }
            *reinterpret_cast<float4*>(&sm.V[r * PV + cc]) = x;
        }
        for (int i = tid; i < DK; i += NT) sm.lam[i] = p.lam[widx * DK + i];
        __syncthreads();

        // X = Kh S^T and Y = Qh S^T (k relabelled to the accumulator rows: step (j, s) takes
        // d_k column 16j + 4lq + s)
        f32x4_t X[4], Y[4], D[4], O[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            X[t] = Y[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKB; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int a = (16 * t + l16) * PK + 16 * j + 4 * lq + s;
                    X[t] = mfma4(sm.Kh[a], ST[j][s], X[t]);
                    Y[t] = mfma4(sm.Qh[a], ST[j][s], Y[t]);
                }
        }
        // R = V - X (in place), Delta = Mmat R, O = Y + P Delta
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) X[t][m] = sm.V[(16 * t + 4 * lq + m) * PV + 16 * wave + l16] - X[t][m];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            D[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
                for (int s = 0; s < 4; ++s) D[t] = mfma4(sm.M[(16 * t + l16) * PC + 16 * t2 + 4 * lq + s], X[t2][s], D[t]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            O[t] = Y[t];
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
                for (int s = 0; s < 4; ++s) O[t] = mfma4(sm.P[(16 * t + l16) * PC + 16 * t2 + 4 * lq + s], D[t2][s], O[t]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * t + 4 * lq + m;
                if (r < len) static_cast<TO*>(p.o)[((bos + r) * H + h) * DV + dvw + l16] = from_f32<TO>(O[t][m]);
            }
        }
        // S^T <- Diag(lam) S^T + Kd^T Delta
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            f32x4_t acc;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = ST[j][m] * sm.lam[16 * j + 4 * lq + m];
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma4(sm.Kd[(16 * t2 + 4 * lq + s) * PK + 16 * j + l16], D[t2][s], acc);
            ST[j] = acc;
        }
    }
    if (p.hT) {
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            *reinterpret_cast<float4*>(p.hT + srow + 16 * j) = make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
    }
}

// ------------------------------------------------------------- stage 2, bf16 inputs (DMA)
// The products of kda_propagate_kernel on the fp16 matrix core (16x16x32, fp32 accumulation),
// with the operands copied global -> LDS by the DMA path of the buffer loads (no registers, no
// conversion), as the scalar-gate stage 2 for bf16 inputs does: stage 1 leaves Kh, Qh, Kd,
// Mmat and P as LDS images (img_off), V stays bf16 and enters only the fp32 residual (times
// the write gate W with decoupled gates: WG). Per work-group: DVT/16 compute waves (16 columns
// each), a DMA wave and, without W, a store wave that writes o from an LDS staging buffer as in
// the scalar-gate kernel; with W (8 KB more per chunk, no room for the staging buffer) the
// compute waves write o themselves, four adjacent lanes covering 16 consecutive columns of a
// token. A chunk's operands take 68.5 KB of LDS (Kd beside Kh; 76.5 KB with W), so the ring is
// two deep: the DMA wave copies chunk c+1 while chunk c is computed and, before the next
// barrier, waits for all of it. The compute waves differ from the
// scalar-gate ones in three places: the residual is V - Kh S^T (Kh carries the decay), the
// state's columns decay by lam one channel each, and K^T of the state update is read from Kd.
template <int DK, int DVT, bool WG>
struct alignas(16) KdaDmaChunk {
    _Float16 Q[64 * DK];    // Qh
    _Float16 K[64 * DK];    // Kh
    _Float16 Kd[64 * DK];
    _Float16 M[64 * 64];    // Mmat
    _Float16 P[64 * 64];
    uint16_t V[64 * DVT];   // bf16, the work-group's d_v columns
    float lam[DK];          // e^{gamma_last} per channel
    float W[WG ? 64 * DVT : 4];  // the write gate of those columns (decoupled gates)
};
// The DMA wave's copies of one chunk: 1 KB blocks of the images, V (and W) rows gathered from
// the inputs (rows past the chunk's end read as zeros), lam.
template <int DK, int DV, int DVT, bool WG>
__device__ __forceinline__ void kda_copy(KdaDmaChunk<DK, DVT, WG>& dst, const ChunkProblem& p, long bos, int len,
                                         long widx, int h, int dv0, int lane) {
    constexpr int NB_K = 64 * DK * 2 / 1024, NB_V = 64 * DVT * 2 / 1024, ROW_V = DVT * 2;
    const int H = p.H;
    const unsigned lo = 16u * lane;
    auto img = [&](const float* base, long elems) {
        return reinterpret_cast<const char*>(reinterpret_cast<const _Float16*>(base) + elems);
    };
    const char* qimg = img(p.qhat, widx * 64 * DK);
    const char* kimg = img(p.khat, widx * 64 * DK);
    const char* dimg = img(p.kdec, widx * 64 * DK);
    const char* mimg = reinterpret_cast<const char*>(static_cast<const _Float16*>(p.mmat) + widx * 4096);
    const char* pimg = reinterpret_cast<const char*>(static_cast<const _Float16*>(p.pmat) + widx * 4096);
    const unsigned vbytes = (unsigned)((len - 1) * H * DV + DVT) * 2;
    const auto vr = make_rsrc(static_cast<const uint16_t*>(p.v) + (bos * H + h) * DV + dv0, vbytes);
    if (lane < DK / 4) dma16g(reinterpret_cast<const char*>(p.lam + widx * DK), lo, dst.lam);
#pragma unroll
    for (int b = 0; b < NB_V; ++b) {
        const int byte = 1024 * b + 16 * lane, r = byte / ROW_V;
        dma16(vr, reinterpret_cast<const char*>(dst.V) + 1024 * b, r * H * DV * 2 + 16 * ((byte % ROW_V) >> 4));
    }
    if constexpr (WG) {
        constexpr int NB_W = 64 * DVT * 4 / 1024, ROW_W = DVT * 4;
        const auto wr = make_rsrc(p.write + (bos * H + h) * DV + dv0, (unsigned)((len - 1) * H * DV + DVT) * 4);
#pragma unroll
        for (int b = 0; b < NB_W; ++b) {
            const int byte = 1024 * b + 16 * lane, r = byte / ROW_W;
            dma16(wr, reinterpret_cast<const char*>(dst.W) + 1024 * b, r * H * DV * 4 + 16 * ((byte % ROW_W) >> 4));
        }
    }
#pragma unroll
    for (int b = 0; b < NB_K; ++b) {
        dma16g(kimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.K) + 1024 * b);
        dma16g(qimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.Q) + 1024 * b);
        dma16g(dimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.Kd) + 1024 * b);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        dma16g(mimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.M) + 1024 * b);
        dma16g(pimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.P) + 1024 * b);
    }
}

template <typename TO, int DK, int DV, int DVT, bool WG>
__global__ __launch_bounds__((DVT / 16 + (WG ? 1 : 2)) * 64) void kda_propagate_dma_kernel(ChunkProblem p) {
    using CH = KdaDmaChunk<DK, DVT, WG>;
    using OS = OStage<TO, DVT>;
    constexpr int NW = DVT / 16;   // compute waves
    constexpr int NKB = DK / 16;   // d_k tiles of the state
    constexpr int NKS = DK / 32;   // 32-wide d_k slices
    constexpr int NTILE = DV / DVT;
    constexpr int NOS = WG ? 1 : 2;  // output staging (unused with W)
    __shared__ CH ch[2];
    __shared__ OS ost[NOS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;

    // (sequence, head) pair and column tile; with a pair count divisible by 8 the tiles of one
    // pair get block ids equal modulo 8 (same XCD, shared L2 for the pair's operators)
    const long NP = (long)p.N * H;
    const long bid = blockIdx.x;
    long slot;
    int tile;
    if (NP % 8 == 0) {
        const long x = bid % 8, i = bid / 8;
        tile = (int)(i % NTILE);
        slot = (i / NTILE) * 8 + x;
    } else {
        slot = bid / NTILE;
        tile = (int)(bid % NTILE);
    }
    // the work-group's (sequence, head) pair: packed sequences are taken longest first (the chunk
    // table's order)
    const int n = p.cu_seqlens ? p.chunk_base[p.N + 1 + (int)(slot / H)] : (int)(slot / H);
    const int h = (int)(slot % H);
    const long pair = (long)n * H + h;
    const int dv0 = tile * DVT;

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    const long cbase = (p.cu_seqlens == nullptr) ? (long)n * p.nc_per_seq : (long)p.chunk_base[n];
    long nchunks = (seos - sbos + 63) / 64;
    if (cbase + nchunks > p.nc_bound) nchunks = max(0L, p.nc_bound - cbase);
    auto chunk_len = [&](long jc) {
        const long l = seos - (sbos + jc * 64);
        return (int)(l < 64 ? l : 64);
    };

    if (wave == NW) {
        // ------------------------------------------------------------------- DMA wave
        auto copy = [&](long jc) {
            kda_copy<DK, DV, DVT, WG>(ch[jc & 1], p, sbos + jc * 64, chunk_len(jc), (cbase + jc) * H + h, h, dv0, lane);
        };
        if (nchunks > 0) copy(0);
        for (long jc = 0; jc < nchunks; ++jc) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            lds_barrier();  // chunk jc's operands are in LDS; chunk jc-1's buffers are free
            if (jc + 1 < nchunks) copy(jc + 1);
        }
        if constexpr (!WG) lds_barrier();
        return;
    }
    if constexpr (!WG) {
        if (wave == NW + 1) {
            // ------------------------------------------------------------- store wave
            // outputs of chunk jc through a resource sized to the valid rows; NV adjacent
            // lanes write one token row's columns (16 bytes each), so an instruction covers
            // 64/NV rows
            auto store_out = [&](const OS& os, long jc) {
                constexpr int E = (int)sizeof(TO), NV = OS::ROWB / 16, RPI = 64 / NV;
                const long obos = sbos + jc * 64;
                const int olen = chunk_len(jc);
                const auto orr = make_rsrc(static_cast<TO*>(p.o) + (obos * H + h) * DV + dv0,
                                           (unsigned)((olen - 1) * H * DV + DVT) * E);
                const int rr = lane / NV, pc = lane % NV;
                u32x4_t piece[NV];
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    piece[i] = *reinterpret_cast<const u32x4_t*>(&os.b[(RPI * i + rr) * OS::PITCH + 16 * pc]);
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    __builtin_amdgcn_raw_buffer_store_b128(piece[i], orr, (RPI * i + rr) * H * DV * E + 16 * pc, 0, 0);
            };
            for (long jc = 0; jc < nchunks; ++jc) {
                lds_barrier();
                if (jc > 0) store_out(ost[(jc - 1) & 1], jc - 1);
            }
            lds_barrier();  // the last chunk's outputs are staged
            if (nchunks > 0) store_out(ost[(nchunks - 1) & 1], nchunks - 1);
            return;
        }
    }

    // ------------------------------------------------------------------- compute waves
    // wave w: columns dv0 + 16w .. +15; lane holds S[dv0 + 16w + l16][16j + 4lq + 0..3] in ST[j]
    const int dvw = dv0 + 16 * wave;
    f32x4_t ST[NKB];
    const long srow = (pair * DV + dvw + l16) * DK + 4 * lq;
    {
        // the initial state through a resource of zero size when there is none (loads read 0)
        const auto hr = make_rsrc(p.h0 ? p.h0 + (pair * DV + dvw) * DK : nullptr, p.h0 ? (unsigned)(16 * DK * 4) : 0u);
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            ST[j] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(hr, (l16 * DK + 4 * lq + 16 * j) * 4, 0, 0));
    }

    constexpr int E = (int)sizeof(TO);
    auto step = [&](const CH& cm, long jc) {
        lds_barrier();  // chunk data in cm
        uint4 MF[4][2], PF[4][2];
        float4 V4[4];
        auto load_mp = [&](const _Float16* src, uint4 (&f)[4][2]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    f[t][hf] = *reinterpret_cast<const uint4*>(&src[img_off<64>(16 * t + l16, 32 * hf + 4 * lq)]);
        };

        // X = Kh S^T [64 tokens x 16 columns] and Y^T = S Qh^T [16 columns x 64 tokens]
        uint4 BS[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) BS[s] = pack_f16_frag(ST[2 * s], ST[2 * s + 1]);
        uint4 KF[2][4], QF[2][4];  // fragments of slice s in [s % 2]
        auto load_xy = [&](int s, uint4 (&kf)[4], uint4 (&qf)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int row = 16 * t + l16, c0 = 32 * s + 4 * lq;
                kf[t] = *reinterpret_cast<const uint4*>(&cm.K[img_off<DK>(row, c0)]);
                qf[t] = *reinterpret_cast<const uint4*>(&cm.Q[img_off<DK>(row, c0)]);
            }
        };
        load_xy(0, KF[0], QF[0]);
        f32x4_t X[4], Y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            X[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            Y[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int b = s & 1;
            if (s + 1 < NKS) {
                load_xy(s + 1, KF[b ^ 1], QF[b ^ 1]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) V4[t] = load4_t<uint16_t>(&cm.V[(16 * t + 4 * lq) * DVT + 16 * wave], DVT);
                load_mp(cm.M, MF);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                X[t] = mfma_f16(KF[b][t], BS[s], X[t]);
                Y[t] = mfma_f16(BS[s], QF[b][t], Y[t]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // R = V - X (W * V - X with decoupled gates);  Delta = Mmat R
        load_mp(cm.P, PF);
        if constexpr (WG) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float* wc = &cm.W[(16 * t + 4 * lq) * DVT + 16 * wave + l16];
                V4[t] = make_float4(V4[t].x * wc[0], V4[t].y * wc[DVT], V4[t].z * wc[2 * DVT], V4[t].w * wc[3 * DVT]);
            }
        }
        f32x4_t R[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            R[t] = f32x4_t{V4[t].x - X[t][0], V4[t].y - X[t][1], V4[t].z - X[t][2], V4[t].w - X[t][3]};
        const uint4 BR[2] = {pack_f16_frag(R[0], R[1]), pack_f16_frag(R[2], R[3])};
        f32x4_t D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) D[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int t = 0; t < 4; ++t) D[t] = mfma_f16(MF[t][hf], BR[hf], D[t]);
        __builtin_amdgcn_sched_barrier(0);

        // Kd^T fragments for the state update, read while the output product runs
        const int tr = l16 >> 2, tc = 4 * (l16 & 3);
        uint4 KT[NKB][2];
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            const int c = 16 * j + tc;
            KT[j][0] = lds_frag2_t(&cm.Kd[img_off<DK>(4 * lq + tr, c)], &cm.Kd[img_off<DK>(16 + 4 * lq + tr, c)]);
            KT[j][1] = lds_frag2_t(&cm.Kd[img_off<DK>(32 + 4 * lq + tr, c)], &cm.Kd[img_off<DK>(48 + 4 * lq + tr, c)]);
        }

        // O^T = S Qh^T + Delta^T P^T (lane: token 16t + l16, columns 16 wave + 4 lq .. +3): staged
        // for the store wave, or with W out through a resource sized to the chunk's valid rows
        const uint4 BD[2] = {pack_f16_frag(D[0], D[1]), pack_f16_frag(D[2], D[3])};
        f32x4_t O[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) O[t] = Y[t];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int t = 0; t < 4; ++t) O[t] = mfma_f16(BD[hf], PF[t][hf], O[t]);
        if constexpr (WG) {
            const auto orr = make_rsrc(static_cast<TO*>(p.o) + ((sbos + jc * 64) * H + h) * DV + dv0,
                                       (unsigned)((chunk_len(jc) - 1) * H * DV + DVT) * E);
#pragma unroll
            for (int t = 0; t < 4; ++t) buf_store4<TO>(orr, ((16 * t + l16) * H * DV + 16 * wave + 4 * lq) * E, O[t]);
        } else {
            OS& os = ost[jc & 1];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                char* dst = &os.b[(16 * t + l16) * OS::PITCH + (16 * wave + 4 * lq) * E];
                if constexpr (E == 2)
                    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(O[t][0], O[t][1]), pack_bf16x2(O[t][2], O[t][3]));
                else
                    *reinterpret_cast<float4*>(dst) = make_float4(O[t][0], O[t][1], O[t][2], O[t][3]);
            }
        }

        // S^T <- Diag(lam) S^T + Kd^T Delta
#pragma unroll
        for (int j = 0; j < NKB; ++j) ST[j] *= *reinterpret_cast<const f32x4_t*>(&cm.lam[16 * j + 4 * lq]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int j = 0; j < NKB; ++j) ST[j] = mfma_f16(KT[j][hf], BD[hf], ST[j]);
    };

    for (long jc = 0; jc < nchunks; ++jc) step(ch[jc & 1], jc);
    if constexpr (!WG) lds_barrier();  // hand the last chunk's outputs to the store wave

    if (p.hT) {
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            *reinterpret_cast<float4*>(p.hT + srow + 16 * j) = make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
    }
}

// -------------------------------------------------------------------- launchers
KdaLayout kda_workspace_layout(int B, int T, int H, int dk, int N, int varlen, int elem) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    KdaLayout w{};
    w.nc_bound = varlen ? ((long)T + (long)N * 63) / 64 : (long)B * (((long)T + 63) / 64);
    const size_t units = (size_t)w.nc_bound * H;
    w.off_base = 0;
    w.off_m = al(varlen ? (size_t)(2 * N + 1) * 4 : 0);   // chunk_base, then the chain order
    w.off_p = al(w.off_m + units * 4096 * elem);
    w.off_kh = al(w.off_p + units * 4096 * elem);
    w.off_qh = al(w.off_kh + units * 64 * dk * elem);
    w.off_kd = al(w.off_qh + units * 64 * dk * elem);
    w.off_lam = al(w.off_kd + units * 64 * dk * elem);
    w.total = w.off_lam + units * dk * 4;
    if (w.nc_bound == 0) w.total = al(varlen ? (size_t)(2 * N + 1) * 4 : 0);
    return w;
}

template <typename TIn, typename TO, int DK, int DV>
static hipError_t kda_launch(const ChunkProblem& p, hipStream_t s) {
    constexpr int DVT = 32;
    const long units = p.nc_bound * p.H;
    hipError_t e = hipSuccess;
    if (units > 0) {
        // persistent grid: as many work-groups as the device holds at once
        auto go = [&](auto kern, std::atomic<int> (&resident)[64]) {
            const long cap = resident_blocks(kern, kKdaPrepThreads, resident, 1);
            return launch(kern, dim3((unsigned)(units < cap ? units : cap)), dim3(kKdaPrepThreads), s, p);
        };
        static std::atomic<int> resident_erase[64], resident_beta[64];
        e = p.erase ? go(kda_prepare_kernel<TIn, DK, true>, resident_erase)
                    : go(kda_prepare_kernel<TIn, DK, false>, resident_beta);
    }
    const long pairs = (long)p.N * p.H;
    if (e != hipSuccess || pairs == 0) return e;
    const dim3 grid((unsigned)(pairs * (DV / DVT)));
    if constexpr (sizeof(TIn) == 2) {
        if (p.write == nullptr)
            return launch(kda_propagate_dma_kernel<TO, DK, DV, DVT, false>, grid, dim3((DVT / 16 + 2) * 64), s, p);
        return launch(kda_propagate_dma_kernel<TO, DK, DV, DVT, true>, grid, dim3((DVT / 16 + 1) * 64), s, p);
    } else {
        return launch(kda_propagate_kernel<TIn, TO, DK, DV, DVT>, grid, dim3(DVT / 16 * 64), s, p);
    }
}

template <typename TIn, typename TO>
static hipError_t kda_dispatch(const ChunkProblem& p, hipStream_t s) {
    if (p.dk == 64)
        return p.dv == 64 ? kda_launch<TIn, TO, 64, 64>(p, s) : kda_launch<TIn, TO, 64, 128>(p, s);
    return p.dv == 64 ? kda_launch<TIn, TO, 128, 64>(p, s) : kda_launch<TIn, TO, 128, 128>(p, s);
}

hipError_t launch_kda_chunk_fwd(const ChunkProblem& p, hipStream_t s) {
    hipError_t e = launch_chunk_base(p, s);
    if (e != hipSuccess) return e;
    if (!p.bf16) return kda_dispatch<float, float>(p, s);
    return p.o_bf16 ? kda_dispatch<uint16_t, uint16_t>(p, s) : kda_dispatch<uint16_t, float>(p, s);
}

}  // namespace gdn
