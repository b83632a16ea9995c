// Chunkwise-parallel forward pass of the gated delta rule for gfx950.
//
// The method (WY representation / UT transform extended to carry the gate) is named in
// the paper note "Gated Delta Networks: Improving Mamba2 with Delta Rule" (phantomic12
// inference-research), mechanism paragraph, and in record "LIT-137"
// (anthology-of-the-sota), "Standing in the anthology". For one chunk of n <= 64 tokens
// entering with state S [d_v, d_k], with gamma the in-chunk cumulative sum of g = log alpha:
//
//   A     = strict_lower(diag(beta) K K^T * exp(gamma_r - gamma_i))     gated Gram
//   T     = (I + A)^{-1}                                                UT transform
//   Mmat  = T diag(beta)             (so U = Mmat V and W = Mmat diag(e^gamma) K)
//   P     = (Q K^T) * exp(gamma_r - gamma_i) * [i <= r]    (read after the write)
//   R     = V - diag(e^gamma) K S^T
//   Delta = Mmat R  (= U - W S^T)                                       effective writes
//   O     = diag(e^gamma) Q S^T + P Delta
//   S'    = e^{gamma_last} S + Delta^T diag(e^{gamma_last - gamma}) K
//
// Stage 1 (chunk_prepare_kernel) computes, for every chunk in parallel, the gate tables
// e^gamma and e^{gamma_last - gamma}, Mmat and P. Stage 2 (chunk_propagate_kernel) walks the
// chunks of one (sequence, head, d_v tile) in order with the fp32 state in registers and
// writes O. Every gate factor is exp of a non-positive difference, masked before the exp.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_stage2.h"
#include "gdn_ut.h"

namespace gdn {

// ------------------------------------------------------------------ chunk table
// base[n] = number of chunks in sequences 0..n-1 (each sequence is cut into 64-token
// chunks from its own start); base[N] = total. Token ranges are clamped to [0, T] so a
// malformed offset array cannot move any later access out of bounds. Then base[N + 1 + k] =
// the k-th sequence in order of decreasing chunk count (ties by index; the identity order
// above 1024 sequences): the state propagation takes the sequences' chains longest first, so
// that a long chain does not start last and extend the launch (its work-groups run one per CU).
__global__ __launch_bounds__(1024) void chunk_base_kernel(const int32_t* __restrict__ cu, int N,
                                                          int T, int32_t* __restrict__ base) {
    __shared__ int32_t part[1024];
    __shared__ int32_t cnt[1024];
    const int tid = threadIdx.x;
    const int per = (N + 1023) / 1024;
    const int s0 = min(N, tid * per), s1 = min(N, s0 + per);
    auto nchunks = [&](int m) {
        const int b0 = min(max(cu[m], 0), T);
        const int b1 = min(max(cu[m + 1], b0), T);
        return (b1 - b0 + kChunk - 1) / kChunk;
    };
    int32_t local = 0;
    for (int m = s0; m < s1; ++m) local += nchunks(m);
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t x = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    int32_t run = part[tid] - local;
    for (int m = s0; m < s1; ++m) {
        base[m] = run;
        run += nchunks(m);
    }
    if (tid == 1023) base[N] = part[1023];
    int32_t* order = base + N + 1;
    if (N > 1024) {
        for (int m = s0; m < s1; ++m) order[m] = m;
        return;
    }
    const int c = tid < N ? nchunks(tid) : 0;
    cnt[tid] = c;
    __syncthreads();
    if (tid < N) {
        int rank = 0;
        for (int m = 0; m < N; ++m) rank += (cnt[m] > c) || (cnt[m] == c && m < tid);
        order[rank] = tid;
    }
}

// ------------------------------------------------------------------- stage 1
template <typename TIn, int DK>
struct alignas(16) PrepSmem {
    using TM = typename Operand<TIn>::type;
    static constexpr int PK = DK + 16 / (int)sizeof(TIn);  // raw K, Q row pitch (elements)
    static constexpr int PC = 64 + 16 / (int)sizeof(TM);   // P row pitch
    static constexpr int PF = 68;                           // fp32 A, T row pitch
    union {
        struct { TIn K[64 * PK]; TIn Q[64 * PK]; } in;
        struct { float A[64 * PF]; float T[64 * PF]; } tri;
    } u;
    TM P[64 * PC];
    TM Plo[sizeof(TM) == 2 ? 64 * PC : 8];   // fp16 operands: P - fp16(P) (backward pass)
    float graw[64];   // g as loaded
    float gam[64];    // its in-chunk inclusive cumulative sum
    float beta[64];
};

// Register staging of one chunk's K, Q, g, beta (raw input elements).
template <typename TIn, int DK>
struct PrepStage {
    static constexpr int EPV = 16 / (int)sizeof(TIn);
    static constexpr int VPR = DK / EPV;
    static constexpr int NV = 64 * VPR / 256;
    uint4 rk[NV], rq[NV];
    float rg, rb;

    __device__ __forceinline__ void load(const ChunkProblem& p, long bos, int len, int h, int tid) {
        const int H = p.H;
        const TIn* kp = static_cast<const TIn*>(p.k);
        const TIn* qp = static_cast<const TIn*>(p.q);
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int vi = tid + 256 * it, r = vi / VPR, cv = vi % VPR;
            rk[it] = zero16();
            rq[it] = zero16();
            if (r < len) {
                const long off = ((bos + r) * H + h) * DK + cv * EPV;
                rk[it] = *reinterpret_cast<const uint4*>(kp + off);
                rq[it] = *reinterpret_cast<const uint4*>(qp + off);
            }
        }
        rg = 0.f;
        rb = 0.f;
        if (tid < len) {
            const long o = (bos + tid) * H + h;
            rg = p.g[o];
            rb = p.beta[o];
        }
    }

    __device__ __forceinline__ void store(PrepSmem<TIn, DK>& sm, int tid) const {
        constexpr int PK = PrepSmem<TIn, DK>::PK;
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int vi = tid + 256 * it, r = vi / VPR, cv = vi % VPR;
            *reinterpret_cast<uint4*>(&sm.u.in.K[r * PK + cv * EPV]) = rk[it];
            *reinterpret_cast<uint4*>(&sm.u.in.Q[r * PK + cv * EPV]) = rq[it];
        }
        if (tid < 64) {
            sm.graw[tid] = rg;
            sm.beta[tid] = rb;
        }
    }
};

// bf16 inputs: the chunk's K and diag(e^gamma) Q as fp16 images [64, DK] (rows past the
// chunk's end zero), from the raw tiles in LDS and the scanned gamma.
template <typename TIn, int DK>
__device__ __forceinline__ void write_kq_images(const PrepSmem<TIn, DK>& sm, _Float16* kimg,
                                                _Float16* qimg, int tid) {
    if constexpr (sizeof(TIn) == 2) {
        constexpr int PK = PrepSmem<TIn, DK>::PK, NI = 64 * DK / 8 / 256;
        auto cvt = [](uint2 a, uint2 b, float e) {
            auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
            auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
            return make_uint4(pack_f16x2(e * lo(a.x), e * hi(a.x)), pack_f16x2(e * lo(a.y), e * hi(a.y)),
                              pack_f16x2(e * lo(b.x), e * hi(b.x)), pack_f16x2(e * lo(b.y), e * hi(b.y)));
        };
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            const int i = tid + 256 * it;
            int r, c0;
            img_piece<DK>(i, r, c0);
            const uint2 ka = *reinterpret_cast<const uint2*>(&sm.u.in.K[r * PK + c0]);
            const uint2 kb = *reinterpret_cast<const uint2*>(&sm.u.in.K[r * PK + c0 + 16]);
            const uint2 qa = *reinterpret_cast<const uint2*>(&sm.u.in.Q[r * PK + c0]);
            const uint2 qb = *reinterpret_cast<const uint2*>(&sm.u.in.Q[r * PK + c0 + 16]);
            reinterpret_cast<uint4*>(kimg)[i] = cvt(ka, kb, 1.f);
            reinterpret_cast<uint4*>(qimg)[i] = cvt(qa, qb, __expf(sm.gam[r]));
        }
    }
}

// Persistent work-groups: each walks (chunk, head) units with a stride of the grid, keeping
// the next unit's inputs in flight in registers while the current one is computed. BWD: the
// instance run by the backward pass, which also keeps T row-major and writes the operators
// for its own kernels (fp32 inputs: fp32 T, Mmat, P row-major and, when set, fp16 copies;
// bf16 inputs: fp16 T row-major and the fp16 images of Mmat, P and P's rounding remainder).
template <typename TIn, int DK, bool BWD>
__global__ __launch_bounds__(256) void chunk_prepare_kernel(ChunkProblem p) {
    using SM = PrepSmem<TIn, DK>;
    using TM = typename SM::TM;
    constexpr int PK = SM::PK, PC = SM::PC, PF = SM::PF;
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;
    const long nunits = p.nc_bound * H;

    PrepStage<TIn, DK> stage;
    long unit = blockIdx.x;
    long bos = 0;
    int len = 0;
    bool ok = unit < nunits && locate_chunk(p, unit / H, bos, len);
    if (ok) stage.load(p, bos, len, (int)(unit % H), tid);

    while (unit < nunits) {
        const long nxt = unit + gridDim.x;
        long nbos = 0;
        int nlen = 0;
        const bool nok = nxt < nunits && locate_chunk(p, nxt / H, nbos, nlen);
        if (ok) {
            const long c = unit / H;
            const int h = (int)(unit % H);
            const long widx = c * H + h;
            __syncthreads();  // the previous unit is done with LDS
            stage.store(sm, tid);
            __syncthreads();
            if (nok) stage.load(p, nbos, nlen, (int)(nxt % H), tid);

            // -- gate scan (every wave scans its own copy, so no barrier is needed before the
            //    reads of gamma below; the identical LDS writes of the four waves are benign) and
            //    gate tables (wave 0)
            {
                const float x = wave_inclusive_sum(sm.graw[lane]);
                sm.gam[lane] = x;
                if (wave == 0) {
                    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
                    p.gates[widx * 128 + lane] = __expf(x);
                    p.gates[widx * 128 + 64 + lane] = __expf(last - x);
                }
            }
            if (p.k16) write_kq_images<TIn, DK>(sm, p.k16 + widx * 64 * DK, p.q16 + widx * 64 * DK, tid);

            // -- K K^T and Q K^T (exact products of the inputs); wave w owns row block w
            const int rb = wave;
            f32x4_t G[4], P0[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                G[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                P0[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                const TIn* brow = &sm.u.in.K[(16 * cb + l16) * PK];
                mma_nt_in<TIn, DK>(G[cb], &sm.u.in.K[(16 * rb + l16) * PK], brow);
                mma_nt_in<TIn, DK>(P0[cb], &sm.u.in.Q[(16 * rb + l16) * PK], brow);
            }
            __syncthreads();  // K and Q are dead; their space becomes A and T

            // -- gate the products: A (strictly lower, fp32) and P (lower incl. diagonal). The
            //    exponent is clamped to <= 0 before the exp, so masked entries cannot overflow.
            {
                const float4 gr = *reinterpret_cast<const float4*>(&sm.gam[16 * rb + 4 * lq]);
                const float4 br = *reinterpret_cast<const float4*>(&sm.beta[16 * rb + 4 * lq]);
                const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, brv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const float gc = sm.gam[16 * cb + l16];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int r = 16 * rb + 4 * lq + v, i = 16 * cb + l16;
                        const float e = __expf(fminf(grv[v] - gc, 0.f));
                        const float a = (i < r) ? brv[v] * G[cb][v] * e : 0.f;
                        const float pp = (i <= r) ? P0[cb][v] * e : 0.f;
                        sm.u.tri.A[r * PF + i] = a;
                        const TM ph = from_f32<TM>(pp);
                        sm.P[r * PC + i] = ph;
                        // backward pass, bf16 inputs: also P's fp16 rounding remainder
                        if constexpr (sizeof(TM) == 2 && BWD) sm.Plo[r * PC + i] = (TM)(pp - (float)ph);
                    }
                }
            }
            __syncthreads();

            // -- T = (I + A)^{-1}
            float* At = sm.u.tri.A;
            float* Tt = sm.u.tri.T;
            ut_inverse64<PF>(At, Tt, wave, lane);

            // -- Mmat = T diag(beta) and P to the workspace: fp32 row-major, fp16 as images
            if constexpr (sizeof(TM) == 4) {
                const int r = tid >> 2, c0 = (tid & 3) * 16;
                float mv[16], pv[16], tv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int ci = c0 + e;
                    tv[e] = ((ci >> 4) <= (r >> 4)) ? Tt[r * PF + ci] : 0.f;
                    mv[e] = tv[e] * sm.beta[ci];
                    pv[e] = to_f32(sm.P[r * PC + ci]);
                }
                store16<TM>(static_cast<TM*>(p.mmat) + widx * 4096 + r * 64 + c0, mv);
                store16<TM>(static_cast<TM*>(p.pmat) + widx * 4096 + r * 64 + c0, pv);
                if (BWD) store16<float>(p.tmat + widx * 4096 + r * 64 + c0, tv);
            } else {
                if constexpr (BWD) {  // backward pass, bf16 inputs: also T, fp16 row-major
                    const int r = tid >> 2, c0 = (tid & 3) * 16;
                    uint32_t tv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int ci = c0 + 2 * e;
                        const bool on = (ci >> 4) <= (r >> 4);   // both columns in one 16-block
                        tv[e] = pack_f16x2(on ? Tt[r * PF + ci] : 0.f, on ? Tt[r * PF + ci + 1] : 0.f);
                    }
                    uint4* tq = reinterpret_cast<uint4*>(p.tmat16 + widx * 4096 + r * 64 + c0);
                    tq[0] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
                    tq[1] = make_uint4(tv[4], tv[5], tv[6], tv[7]);
                }
                // the backward pass takes the images from mimg16, pimg16 and adds that of P's
                // rounding remainder (plo16)
                _Float16* mimg = BWD ? p.mimg16 : static_cast<TM*>(p.mmat);
                _Float16* pimg = BWD ? p.pimg16 : static_cast<TM*>(p.pmat);
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const int i = tid + 256 * it;
                    int r, c0;
                    img_piece<64>(i, r, c0);
                    float mv[8], pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int ci = c0 + (e & 3) + 16 * (e >> 2);
                        mv[e] = ((ci >> 4) <= (r >> 4)) ? Tt[r * PF + ci] * sm.beta[ci] : 0.f;
                        pv[e] = to_f32(sm.P[r * PC + ci]);
                    }
                    reinterpret_cast<uint4*>(mimg + widx * 4096)[i] =
                        make_uint4(pack_f16x2(mv[0], mv[1]), pack_f16x2(mv[2], mv[3]),
                                   pack_f16x2(mv[4], mv[5]), pack_f16x2(mv[6], mv[7]));
                    reinterpret_cast<uint4*>(pimg + widx * 4096)[i] =
                        make_uint4(pack_f16x2(pv[0], pv[1]), pack_f16x2(pv[2], pv[3]),
                                   pack_f16x2(pv[4], pv[5]), pack_f16x2(pv[6], pv[7]));
                    if constexpr (BWD) {
                        const uint2 la = *reinterpret_cast<const uint2*>(&sm.Plo[r * PC + c0]);
                        const uint2 lb = *reinterpret_cast<const uint2*>(&sm.Plo[r * PC + c0 + 16]);
                        reinterpret_cast<uint4*>(p.plo16 + widx * 4096)[i] = make_uint4(la.x, la.y, lb.x, lb.y);
                    }
                }
            }
        } else if (nok) {
            stage.load(p, nbos, nlen, (int)(nxt % H), tid);
        }
        unit = nxt;
        ok = nok;
    }
}

// ------------------------------------------------------------------- stage 2
template <typename TIn, int DK, int DVT>
struct alignas(16) PropSmem {
    using TM = typename Operand<TIn>::type;
    static constexpr int PK = KQLayout<TM, DK>::kPitch;    // K, Q row pitch (operand type)
    static constexpr int PC = 64 + 16 / (int)sizeof(TM);   // Mmat, P row pitch
    static constexpr int PV = DVT + 32 / (int)sizeof(TIn); // V tile row pitch (raw input)
    TM K[64 * PK];
    TM Q[64 * PK];
    TM M[64 * PC];
    TM P[64 * PC];
    TIn V[64 * PV];
    float eg[64];   // e^{gamma_r}
    float ed[64];   // e^{gamma_last - gamma_r}
};

// Global -> register -> LDS staging of one chunk's inputs, so that the loads for chunk c+1
// are in flight while chunk c is computed. K and Q are converted to the operand type on the
// way into LDS; V stays in the input type (it is only used elementwise).
template <typename TIn, int DK, int DV, int DVT>
struct PropStage {
    using TM = typename Operand<TIn>::type;
    using SM = PropSmem<TIn, DK, DVT>;
    using KL = KQLayout<TM, DK>;
    static constexpr int NT = DVT / 16 * 64;                // threads
    static constexpr int EPV = 16 / (int)sizeof(TIn);
    static constexpr int VPR_K = DK / EPV, NV_K = 64 * VPR_K / NT;
    static constexpr int VPR_V = DVT / EPV, NV_V = 64 * VPR_V / NT;
    static constexpr int EPM = 16 / (int)sizeof(TM);
    static constexpr int VPR_M = 64 / EPM, NV_M = 64 * VPR_M / NT;
    static_assert(NV_K * NT == 64 * VPR_K && NV_V * NT == 64 * VPR_V && NV_M * NT == 64 * VPR_M,
                  "staging shape");
    uint4 rk[NV_K], rq[NV_K], rv[NV_V], rm[NV_M], rp[NV_M];
    float4 rgt;

    // Loads chunk (first token bos, len tokens) of head h; rows past len read as zeros. The
    // loads are numbered in a fixed order and only those with number % nparts == part are
    // issued, so that a caller can spread them over its compute (part and nparts fold to
    // constants where the caller's loop is unrolled).
    __device__ __forceinline__ void load(const ChunkProblem& p, long bos, int len, long widx, int h,
                                         int dv0, int tid, int part = 0, int nparts = 1) {
        const int H = p.H;
        const long tok0 = bos * H + h;
        constexpr int E = (int)sizeof(TIn);
        const unsigned kbytes = (unsigned)((len - 1) * H * DK + DK) * E;
        const unsigned vbytes = (unsigned)((len - 1) * H * DV + DVT) * E;
        const auto kr = make_rsrc(static_cast<const TIn*>(p.k) + tok0 * DK, kbytes);
        const auto qr = make_rsrc(static_cast<const TIn*>(p.q) + tok0 * DK, kbytes);
        const auto vr = make_rsrc(static_cast<const TIn*>(p.v) + tok0 * DV + dv0, vbytes);
        int n = 0;
#pragma unroll
        for (int it = 0; it < NV_K; ++it) {
            const int vi = tid + NT * it, r = vi / VPR_K, cv = vi % VPR_K;
            const int off = (r * H * DK + cv * EPV) * E;
            if (n++ % nparts == part) rk[it] = buf_load16(kr, off);
            if (n++ % nparts == part) rq[it] = buf_load16(qr, off);
        }
#pragma unroll
        for (int it = 0; it < NV_V; ++it) {
            const int vi = tid + NT * it, r = vi / VPR_V, cv = vi % VPR_V;
            if (n++ % nparts == part) rv[it] = buf_load16(vr, (r * H * DV + cv * EPV) * E);
        }
        const uint4* mp = reinterpret_cast<const uint4*>(static_cast<const TM*>(p.mmat) + widx * 4096);
        const uint4* pp = reinterpret_cast<const uint4*>(static_cast<const TM*>(p.pmat) + widx * 4096);
#pragma unroll
        for (int it = 0; it < NV_M; ++it) {
            if (n++ % nparts == part) rm[it] = mp[tid + NT * it];
            if (n++ % nparts == part) rp[it] = pp[tid + NT * it];
        }
        if (n % nparts == part) rgt = reinterpret_cast<const float4*>(p.gates + widx * 128)[tid & 31];
    }

    __device__ __forceinline__ void store(SM& sm, int tid) const {
#pragma unroll
        for (int it = 0; it < NV_K; ++it) {
            const int vi = tid + NT * it, r = vi / VPR_K, cv = vi % VPR_K;
            const int o = KL::off(r, cv * EPV);
            *reinterpret_cast<uint4*>(&sm.K[o]) = to_operand16<TIn>(rk[it]);
            *reinterpret_cast<uint4*>(&sm.Q[o]) = to_operand16<TIn>(rq[it]);
        }
#pragma unroll
        for (int it = 0; it < NV_V; ++it) {
            const int vi = tid + NT * it, r = vi / VPR_V, cv = vi % VPR_V;
            *reinterpret_cast<uint4*>(&sm.V[r * SM::PV + cv * EPV]) = rv[it];
        }
#pragma unroll
        for (int it = 0; it < NV_M; ++it) {
            const int vi = tid + NT * it, r = vi / VPR_M, cv = vi % VPR_M;
            *reinterpret_cast<uint4*>(&sm.M[r * SM::PC + cv * EPM]) = rm[it];
            *reinterpret_cast<uint4*>(&sm.P[r * SM::PC + cv * EPM]) = rp[it];
        }
        if (tid < 32) reinterpret_cast<float4*>(sm.eg)[tid] = rgt;  // eg then ed, contiguous
    }
};

// One work-group per (sequence, head, d_v tile of DVT columns); wave w owns the 16 columns
// dv0 + 16w .. +15 for all 64 tokens of every chunk, so the waves only meet at the input
// staging. The state is held transposed, S^T [d_k, 16], as d_k/16 accumulator tiles (lane
// holds S[dv0 + 16w + l16][16j + 4*lq + 0..3]). Each product's accumulator feeds the next
// product's right operand directly from registers (pack_frag); only the left operands (rows
// of K, Q, Mmat, P, and K^T through transposing reads) come from LDS. A chunk's outputs are
// written at the start of the next chunk, before its prefetch, so that waiting for the
// prefetched inputs never waits for output stores.
template <typename TIn, typename TO, int DK, int DV, int DVT>
__global__ __launch_bounds__(DVT / 16 * 64) void chunk_propagate_kernel(ChunkProblem p) {
    using SM = PropSmem<TIn, DK, DVT>;
    using TM = typename SM::TM;
    using KL = KQLayout<TM, DK>;
    constexpr int PC = SM::PC, PV = SM::PV;
    constexpr int NKB = DK / 16;   // d_k tiles of the state
    constexpr int NKS = DK / 32;   // 32-wide d_k slices
    constexpr int NTILE = DV / DVT;
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;

    // (sequence, head) pair and d_v tile. When the pair count allows it, the NTILE tiles
    // of one pair get block ids that are equal modulo 8, i.e. land on the same XCD and
    // share its L2 for K, Q, Mmat and P.
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
    const int dvw = dv0 + 16 * wave;  // this wave's first d_v column

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    const long cbase = (p.cu_seqlens == nullptr) ? (long)n * p.nc_per_seq : (long)p.chunk_base[n];
    long nchunks = (seos - sbos + kChunk - 1) / kChunk;
    if (cbase + nchunks > p.nc_bound) nchunks = max(0L, p.nc_bound - cbase);

    // -- state S^T in accumulator tiles
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

    PropStage<TIn, DK, DV, DVT> stage;
    auto chunk_len = [&](long jc) {
        const long l = seos - (sbos + jc * kChunk);
        return (int)(l < kChunk ? l : kChunk);
    };
    if (nchunks > 0) stage.load(p, sbos, chunk_len(0), cbase * H + h, h, dv0, tid);
    // Outputs of the previous chunk, transposed (lane holds o[token 16t + l16][dvw + 4lq + v]),
    // written one iteration late through a resource sized to the chunk's valid rows.
    f32x4_t O[4];
    long obos = 0;
    int olen = 0;
    auto store_out = [&]() {
        constexpr int E = (int)sizeof(TO);
        const auto orr = make_rsrc(static_cast<TO*>(p.o) + (obos * H + h) * DV,
                                   (unsigned)((olen - 1) * H * DV + DV) * E);
#pragma unroll
        for (int t = 0; t < 4; ++t) buf_store4<TO>(orr, ((16 * t + l16) * H * DV + dvw + 4 * lq) * E, O[t]);
    };

    for (long jc = 0; jc < nchunks; ++jc) {
        __syncthreads();  // every wave is done with the previous chunk's LDS data
        stage.store(sm, tid);
        __syncthreads();
        if (jc > 0 && p.o) store_out();
        // the next chunk's loads are issued a quarter at a time between the token tiles below
        const bool more = jc + 1 < nchunks;
        const long nbos = sbos + (jc + 1) * kChunk, nwidx = (cbase + jc + 1) * H + h;
        const int nlen = more ? chunk_len(jc + 1) : 1;

        if (p.states) {  // the state entering this chunk, for the backward pass
            float* sp = p.states + (((cbase + jc) * H + h) * DV + dvw + l16) * DK + 4 * lq;
#pragma unroll
            for (int j = 0; j < NKB; ++j)
                *reinterpret_cast<float4*>(sp + 16 * j) = make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
        }
        // X = K S^T and Y = Q S^T: [64 tokens x 16 columns] as 4 token tiles
        Frag<TM> BS[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) BS[s] = pack_frag<TM>(ST[2 * s], ST[2 * s + 1]);
        // Y^T = S Q^T is computed transposed ([16 columns x 64 tokens]) so that the output
        // lands as runs of 4 consecutive columns per lane.
        f32x4_t X[4], Y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (more) stage.load(p, nbos, nlen, nwidx, h, dv0, tid, t, 4);
            X[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            Y[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int row = 16 * t + l16;
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int c0 = 32 * s + 4 * lq, c1 = c0 + 16;
                mma_k32(X[t], load_frag2<TM>(&sm.K[KL::off(row, c0)], &sm.K[KL::off(row, c1)]), BS[s]);
                mma_k32(Y[t], BS[s], load_frag2<TM>(&sm.Q[KL::off(row, c0)], &sm.Q[KL::off(row, c1)]));
            }
        }

        // R = V - e^gamma X (fp32); Y^T scaled by e^gamma (one token per lane) for the output
        f32x4_t R[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 eg = *reinterpret_cast<const float4*>(&sm.eg[16 * t + 4 * lq]);
            const float4 v4 = load4_t<TIn>(&sm.V[(16 * t + 4 * lq) * PV + 16 * wave], PV);
            R[t] = f32x4_t{v4.x - eg.x * X[t][0], v4.y - eg.y * X[t][1], v4.z - eg.z * X[t][2],
                           v4.w - eg.w * X[t][3]};
            Y[t] *= sm.eg[16 * t + l16];
        }

        // Delta = Mmat R  (contraction over the chunk's tokens)
        const Frag<TM> BR0 = pack_frag<TM>(R[0], R[1]), BR1 = pack_frag<TM>(R[2], R[3]);
        f32x4_t D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            D[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const TM* mrow = &sm.M[(16 * t + l16) * PC + 4 * lq];
            mma_k32(D[t], load_frag2<TM>(mrow, mrow + 16), BR0);
            mma_k32(D[t], load_frag2<TM>(mrow + 32, mrow + 48), BR1);
        }

        // O^T = e^gamma S Q^T + Delta^T P^T (kept in registers until the next iteration)
        const Frag<TM> BD0 = pack_frag<TM>(D[0], D[1]), BD1 = pack_frag<TM>(D[2], D[3]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            O[t] = Y[t];
            const TM* prow = &sm.P[(16 * t + l16) * PC + 4 * lq];
            mma_k32(O[t], BD0, load_frag2<TM>(prow, prow + 16));
            mma_k32(O[t], BD1, load_frag2<TM>(prow + 32, prow + 48));
        }
        obos = sbos + jc * kChunk;
        olen = chunk_len(jc);

        // S^T <- e^{gamma_last} S^T + K^T diag(e^{gamma_last - gamma}) Delta
        f32x4_t Dd[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 ed = *reinterpret_cast<const float4*>(&sm.ed[16 * t + 4 * lq]);
            Dd[t] = f32x4_t{ed.x * D[t][0], ed.y * D[t][1], ed.z * D[t][2], ed.w * D[t][3]};
        }
        const Frag<TM> BT0 = pack_frag<TM>(Dd[0], Dd[1]), BT1 = pack_frag<TM>(Dd[2], Dd[3]);
        const float elast = sm.eg[63];
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            f32x4_t acc = ST[j] * elast;
            mma_k32(acc, load_kt<TM, DK>(sm.K, 4 * lq, 16 + 4 * lq, j), BT0);
            mma_k32(acc, load_kt<TM, DK>(sm.K, 32 + 4 * lq, 48 + 4 * lq, j), BT1);
            ST[j] = acc;
        }
    }
    if (nchunks > 0 && p.o) store_out();

    if (p.hT) {
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            *reinterpret_cast<float4*>(p.hT + srow + 16 * j) = make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
    }
}

// ------------------------------------------------------- stage 2, bf16 inputs (DMA)
// Stage 2 for bf16 inputs. Each chunk's operands are copied global -> LDS by the DMA path of
// the buffer loads (no registers, no conversion), double-buffered so that chunk c+1 is in
// flight while chunk c is computed, with one barrier per chunk. Stage 1 leaves every matrix
// operand in fp16 (K, diag(e^gamma) Q, Mmat, P; rows past the chunk's end zero); V stays bf16
// and enters only the fp32 residual. All products run on the fp16 matrix core.
//
// K, Q, Mmat and P arrive as the LDS images stage 1 wrote (see img_off); V rows are copied
// as they are, with rows past the chunk's end read as zeros.
// A chunk's operands in LDS, in two parts with different lifetimes: Q is copied one chunk
// ahead (double-buffered), the rest two chunks ahead (triple-buffered).
template <int DK>
struct alignas(16) KQChunk {
    _Float16 Q[64 * DK];   // diag(e^gamma) Q
};
template <int DK, int DVT>
struct alignas(16) MPVChunk {
    _Float16 K[64 * DK];
    _Float16 M[64 * 64];   // Mmat
    _Float16 P[64 * 64];
    uint16_t V[64 * DVT];  // bf16, the work-group's d_v columns
    float eg[64];          // e^{gamma_r}
    float ed[64];          // e^{gamma_last - gamma_r}
};

// The DMA wave's copies for one chunk, as 1 KB DMA blocks: the Q image (copy_kq), and the K
// image, Mmat, P (not when WP is false: the state chain alone needs no P), the gate tables and
// V (copy_mpv; V rows gathered from the input, rows past the chunk's end read as zeros).
// copy_mpv issues kMpvCopies instructions.
template <int DK>
__device__ __forceinline__ void copy_kq(KQChunk<DK>& dst, const ChunkProblem& p, long widx, int lane) {
    constexpr int NB_KQ = 64 * DK * 2 / 1024;
    const unsigned lo = 16u * lane;
    const char* qimg = reinterpret_cast<const char*>(p.q16 + widx * 64 * DK);
#pragma unroll
    for (int b = 0; b < NB_KQ; ++b) dma16g(qimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.Q) + 1024 * b);
}
template <int DK, int DVT, bool WP = true>
constexpr int kMpvCopies = 64 * DK * 2 / 1024 + 8 + (WP ? 8 : 0) + 64 * DVT * 2 / 1024 + 1;
// PART selects the instructions issued: 0 all, 1 the gate tables, V and the K image, 2 Mmat and
// P (issued in that order, PART 1 then PART 2 is the same sequence as PART 0).
template <int DK, int DV, int DVT, bool WP = true, int PART = 0>
__device__ __forceinline__ void copy_mpv(MPVChunk<DK, DVT>& dst, const ChunkProblem& p, long bos, int len,
                                         long widx, int h, int dv0, int lane) {
    constexpr int NB_KQ = 64 * DK * 2 / 1024, NB_V = 64 * DVT * 2 / 1024, ROW_V = DVT * 2;
    const int H = p.H;
    const unsigned lo = 16u * lane;
    const char* mimg = reinterpret_cast<const char*>(static_cast<const _Float16*>(p.mmat) + widx * 4096);
    const char* pimg = reinterpret_cast<const char*>(static_cast<const _Float16*>(p.pmat) + widx * 4096);
    const unsigned vbytes = (unsigned)((len - 1) * H * DV + DVT) * 2;
    const auto vr = make_rsrc(static_cast<const uint16_t*>(p.v) + (bos * H + h) * DV + dv0, vbytes);
    const char* kimg = reinterpret_cast<const char*>(p.k16 + widx * 64 * DK);
    if constexpr (PART != 2) {
        if (lane < 32) dma16g(reinterpret_cast<const char*>(p.gates + widx * 128), lo, dst.eg);
#pragma unroll
        for (int b = 0; b < NB_V; ++b) {
            const int byte = 1024 * b + 16 * lane, r = byte / ROW_V;
            dma16(vr, reinterpret_cast<const char*>(dst.V) + 1024 * b, r * H * DV * 2 + 16 * ((byte % ROW_V) >> 4));
        }
#pragma unroll
        for (int b = 0; b < NB_KQ; ++b) dma16g(kimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.K) + 1024 * b);
    }
    if constexpr (PART != 1) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            dma16g(mimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.M) + 1024 * b);
            if constexpr (WP) dma16g(pimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.P) + 1024 * b);
        }
    }
}

// One work-group per (sequence, head, DVT-column tile) with DVT/16 compute waves (DVT = 64: one
// on every SIMD) and one DMA wave. Compute wave w owns columns dv0 + 16w .. +15 for all tokens,
// with the state S^T [d_k, 16] in d_k/16 accumulator tiles (lane holds
// S[dv0 + 16w + l16][16j + 4*lq + 0..3]); it reads LDS, runs the matrix and vector units and
// writes its outputs straight to global memory with buffer stores that drop the rows past a
// chunk's end (it never waits for them; a wave that has no copies of its own in flight can pass
// the barrier with stores outstanding), the state entering each chunk in fp16 for the backward
// pass's recompute (p.states16; there p.o is NULL), and the records of the long-chain split
// below. While chunk c is computed the DMA wave copies Q of chunk c+1 and the rest of chunk c+2
// into ring buffers (2 and 3 deep: memory latency is about one chunk's compute time), and before
// the next barrier waits for exactly the copies chunk c+1 needs. One barrier per chunk.
// LDS bandwidth bounds this loop: every compute wave reads the chunk's K, Q, Mmat, P and K^T
// from LDS, about 64 KB per chunk.
// The products are those of the generic stage-2 kernel (chunk_propagate_kernel).
//
// Long chains (few sequence-head pairs, many chunks) leave most of the device idle, so SEG
// cuts each sequence's chunks into p.seg_n segments of p.seg_len chunks:
//   SEG = 1: one work-group per (pair, tile, segment); segment 0 starts from h0, the others
//     from a zero state. Each records its final state in p.segst, segments past the first also
//     their states at segment offsets 1, 2, 4, .., and writes o for all its chunks.
//   SEG = 2: one work-group per (pair, tile, segment g >= 1) reruns segment g from the final
//     state SEG = 1 left for segment g-1. After the chunk that ends at a recorded offset it
//     compares its state with the one SEG = 1 recorded there, bit for bit; once they are equal,
//     every later chunk of the segment computed in SEG = 1 saw exactly the state this rerun
//     would give it (the chunk step is a fixed function of its inputs), so the rerun rewrites o
//     only up to that point. Without a match it runs to the segment's end and keeps its final
//     state. It counts the chunks it computed (fewer than the segment's length: it matched).
//   SEG = 3: one work-group per (pair, tile) walks the segments in order. Segment g's SEG = 2
//     rerun started from the true state when every segment before it matched (then the final
//     state of g-1 is the one SEG = 1 left); the walk accepts those, and from the first segment
//     that did not match it carries the true state itself and reruns the following segments as
//     SEG = 2 does, until one matches again. It writes hT.
//   o and hT equal those of the unsplit kernel bit for bit. The saving comes from decay: a
//   segment's dependence on its entering state shrinks by the product of its gates, and once
//   that falls under fp32 rounding the two states agree and all segments are fixed at once.
// OUT = false (the backward pass's state recompute, SEG = 0): the state chain alone; the
// products that only form o (Q S^T, P Delta) and their LDS reads are left out.
template <typename TO, int DK, int DV, int DVT, int SEG, bool OUT = true>
__global__ __launch_bounds__((DVT / 16 + 1) * 64) void chunk_propagate_bf16_kernel(ChunkProblem p) {
    static_assert(OUT || SEG == 0, "the state recompute runs unsplit");
    using KQ = KQChunk<DK>;
    using MPV = MPVChunk<DK, DVT>;
    constexpr int NW = DVT / 16;   // compute waves
    constexpr int NKB = DK / 16;   // d_k tiles of the state
    constexpr int NKS = DK / 32;   // 32-wide d_k slices
    constexpr int NTILE = DV / DVT;
    __shared__ KQ kq[2];
    __shared__ MPV mpv[3];
    __shared__ int match[2][NW];   // SEG >= 2: per compute wave, state equal to the record (by chunk parity)
    constexpr bool CMP = SEG >= 2;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;

    // work unit (pair, or pair and segment) and column tile; with a unit count divisible by 8
    // the tiles of one unit get block ids equal modulo 8 (same XCD, shared L2 for K, Q, Mmat and P)
    const long NP = (long)p.N * H;
    const long NU = SEG == 1 ? NP * p.seg_n : SEG == 2 ? NP * (p.seg_n - 1) : NP;
    const long bid = blockIdx.x;
    long unit;
    int tile;
    if (NU % 8 == 0) {
        const long x = bid % 8, i = bid / 8;
        tile = (int)(i % NTILE);
        unit = (i / NTILE) * 8 + x;
    } else {
        unit = bid / NTILE;
        tile = (int)(bid % NTILE);
    }
    // the work-group's (sequence, head) pair: packed sequences are taken longest first (the chunk
    // table's order; every pass of the split maps its slots the same way)
    const long slot = SEG == 1 ? unit / p.seg_n : SEG == 2 ? unit / (p.seg_n - 1) : unit;
    const int seg = SEG == 1 ? (int)(unit % p.seg_n) : SEG == 2 ? 1 + (int)(unit % (p.seg_n - 1)) : 0;
    const int n = p.cu_seqlens ? p.chunk_base[p.N + 1 + (int)(slot / H)] : (int)(slot / H);
    const int h = (int)(slot % H);
    const long pair = (long)n * H + h;
    const int dv0 = tile * DVT;

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    const long cbase = (p.cu_seqlens == nullptr) ? (long)n * p.nc_per_seq : (long)p.chunk_base[n];
    long nchunks = (seos - sbos + kChunk - 1) / kChunk;
    if (cbase + nchunks > p.nc_bound) nchunks = max(0L, p.nc_bound - cbase);
    auto chunk_len = [&](long jc) {
        const long l = seos - (sbos + jc * kChunk);
        return (int)(l < kChunk ? l : kChunk);
    };
    // chunk range [c0, c0 + len) of segment g
    auto seg_range = [&](int g, long& c0, long& len) {
        c0 = (long)g * p.seg_len;
        len = max(0L, min((long)p.seg_len, nchunks - c0));
    };
    long c_first = 0, c_count = nchunks;   // SEG 0, 1, 2: the work-group's one range
    if constexpr (SEG == 1 || SEG == 2) {
        seg_range(seg, c_first, c_count);
        if (seg > 0 && c_count == 0) return;   // the whole work-group leaves
    }
    // p.segst slot of (segment g, recorded offset, SEG = 1's final state (slot ncp) or SEG = 2's
    // final state without a match (slot ncp + 1)) for this pair
    const int nslot = p.seg_ncp + 2;
    // after the state records: per (pair, tile, segment) the chunks SEG = 2 computed (int32)
    int* reran = reinterpret_cast<int*>(p.segst + NP * p.seg_n * nslot * (long)DV * DK) + (pair * NTILE + tile) * p.seg_n;
    auto seg_state = [&](int g, int slot) { return p.segst + ((pair * p.seg_n + g) * nslot + slot) * (long)DV * DK; };
    // a range ends at the barrier after its last chunk, or (SEG >= 2) at the barrier after a chunk
    // whose end state matched the record; all waves read the same flags after the same barrier
    auto range_done = [&](int i, long len) {
        if (i == len) return true;
        if constexpr (CMP) {
            if (i > 0) {
                bool all = true;
#pragma unroll
                for (int w = 0; w < NW; ++w) all = all && match[(i - 1) & 1][w] != 0;
                return all;
            }
        }
        return false;
    };
    // offset o (1 <= o < len) has a record when it is a power of two
    auto recorded = [](int o, long len) { return o < len && (o & (o - 1)) == 0; };

    if (wave == NW) {
        // ------------------------------------------------------------------- DMA wave
        // Issue order: KQ(0) MPV(0) MPV(1), then per chunk c: KQ(c+1) MPV(c+2) (no KQ without
        // OUT). Loads complete in issue order, so at the top of chunk c only MPV(c+1) may still
        // be in flight.
        auto run = [&](long c0, long len) -> int {
            auto mpv_copy = [&](int i) {
                const long jc = c0 + i;
                copy_mpv<DK, DV, DVT, OUT>(mpv[i % 3], p, sbos + jc * kChunk, chunk_len(jc), (cbase + jc) * H + h, h,
                                      dv0, lane);
            };
            if (len > 0) {
                if constexpr (OUT) copy_kq<DK>(kq[0], p, (cbase + c0) * H + h, lane);
                mpv_copy(0);
            }
            if (len > 1) mpv_copy(1);
            for (int i = 0;; ++i) {
                if (i + 1 < len) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kMpvCopies<DK, DVT, OUT>));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                // chunk i's operands are in LDS; chunk i-1's buffers are free. The barrier has no
                // fence: a release fence would make the compiler wait here for every copy in flight
                // (copies write LDS), where the counts above wait for exactly the ones chunk i needs
                lds_barrier_lgkm();
                if (range_done(i, len)) {
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // copies of an abandoned chunk
                    return i;
                }
                if (OUT && i + 1 < len) copy_kq<DK>(kq[(i + 1) & 1], p, (cbase + c0 + i + 1) * H + h, lane);
                if (i + 2 < len) mpv_copy(i + 2);
            }
        };
        if constexpr (SEG == 3) {   // the same walk as the compute waves'
            // segments before the first stop were fixed by the second pass; from an unfixed one on,
            // the walk reruns segments until one matches its record again
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
        return;
    }
    // ------------------------------------------------------------------- compute waves
    const int dvw = dv0 + 16 * wave;
    f32x4_t ST[NKB];
    const long scol = (dvw + l16) * DK + 4 * lq;   // this lane's offset in a [dv, dk] state
    auto load_state = [&](const float* src) {
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            const float4 x = *reinterpret_cast<const float4*>(src + scol + 16 * j);
            ST[j] = f32x4_t{x.x, x.y, x.z, x.w};
        }
    };
    auto store_state = [&](float* dst) {
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            *reinterpret_cast<float4*>(dst + scol + 16 * j) = make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
    };
    if (SEG == 2) {
        load_state(seg_state(seg - 1, p.seg_ncp));
    } else if (p.h0 && seg == 0 && SEG != 3) {   // SEG = 3 loads states where its walk needs them
        load_state(p.h0 + pair * DV * DK);
    } else {
#pragma unroll
        for (int j = 0; j < NKB; ++j) ST[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // LDS operands are read ahead of the products that use them (the X/Y fragments one
    // 32-wide slice ahead, Mmat and the residual terms in the last slice, P during the
    // residual, K^T during the output product), and each product phase cycles over
    // independent accumulators; the scheduling fences keep that order.
    auto step = [&](const KQ& ck, const MPV& cm, long jc) {  // chunk jc, after its barrier
        uint4 MF[4][2], PF[4][2];
        float4 V4[4], EG4[4];
        auto load_mp = [&](const _Float16* src, uint4 (&f)[4][2]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    f[t][hf] = *reinterpret_cast<const uint4*>(&src[img_off<64>(16 * t + l16, 32 * hf + 4 * lq)]);
        };
        auto load_r = [&]() {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                V4[t] = load4_t<uint16_t>(&cm.V[(16 * t + 4 * lq) * DVT + 16 * wave], DVT);
                EG4[t] = *reinterpret_cast<const float4*>(&cm.eg[16 * t + 4 * lq]);
            }
        };

        // X = K S^T [64 tokens x 16 columns] and Y^T = S (diag(e^gamma) Q)^T [16 columns x 64 tokens]
        uint4 BS[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) BS[s] = pack_f16_frag(ST[2 * s], ST[2 * s + 1]);
        uint4 KF[2][4], QF[2][4];  // fragments of slice s in [s % 2]
        auto load_xy = [&](int s, uint4 (&kf)[4], uint4 (&qf)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int row = 16 * t + l16, c0 = 32 * s + 4 * lq;
                kf[t] = *reinterpret_cast<const uint4*>(&cm.K[img_off<DK>(row, c0)]);
                if constexpr (OUT) qf[t] = *reinterpret_cast<const uint4*>(&ck.Q[img_off<DK>(row, c0)]);
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
            if (s + 1 < NKS) load_xy(s + 1, KF[b ^ 1], QF[b ^ 1]);
            else {
                load_r();
                load_mp(cm.M, MF);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                X[t] = mfma_f16(KF[b][t], BS[s], X[t]);
                if constexpr (OUT) Y[t] = mfma_f16(BS[s], QF[b][t], Y[t]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // R = V - e^gamma X
        if constexpr (OUT) load_mp(cm.P, PF);
        f32x4_t R[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            R[t] = f32x4_t{V4[t].x - EG4[t].x * X[t][0], V4[t].y - EG4[t].y * X[t][1],
                           V4[t].z - EG4[t].z * X[t][2], V4[t].w - EG4[t].w * X[t][3]};

        // Delta = Mmat R
        const uint4 BR[2] = {pack_f16_frag(R[0], R[1]), pack_f16_frag(R[2], R[3])};
        f32x4_t D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) D[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int t = 0; t < 4; ++t) D[t] = mfma_f16(MF[t][hf], BR[hf], D[t]);
        __builtin_amdgcn_sched_barrier(0);

        // K^T fragments for the state update, read while the output product runs
        const int tr = l16 >> 2, tc = 4 * (l16 & 3);
        uint4 KT[NKB][2];
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            const int c = 16 * j + tc;
            KT[j][0] = lds_frag2_t(&cm.K[img_off<DK>(4 * lq + tr, c)], &cm.K[img_off<DK>(16 + 4 * lq + tr, c)]);
            KT[j][1] = lds_frag2_t(&cm.K[img_off<DK>(32 + 4 * lq + tr, c)], &cm.K[img_off<DK>(48 + 4 * lq + tr, c)]);
        }

        // O^T = e^gamma S Q^T + Delta^T P^T (lane: token 16t + l16, columns 16 wave + 4 lq .. +3),
        // stored through a resource that ends at the chunk's last token row
        if constexpr (OUT) {
            const uint4 BD[2] = {pack_f16_frag(D[0], D[1]), pack_f16_frag(D[2], D[3])};
            f32x4_t O[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) O[t] = Y[t];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int t = 0; t < 4; ++t) O[t] = mfma_f16(BD[hf], PF[t][hf], O[t]);
            if (p.o) {
                constexpr int E = (int)sizeof(TO);
                const long obos = sbos + jc * kChunk;
                const auto orr = make_rsrc(static_cast<TO*>(p.o) + (obos * H + h) * DV + dvw,
                                           (unsigned)(((chunk_len(jc) - 1) * H * DV + 16) * E));
#pragma unroll
                for (int t = 0; t < 4; ++t) buf_store4<TO>(orr, ((16 * t + l16) * H * DV + 4 * lq) * E, O[t]);
            }
        }

        // S^T <- e^{gamma_last} S^T + K^T diag(e^{gamma_last - gamma}) Delta
        f32x4_t Dd[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 ed = *reinterpret_cast<const float4*>(&cm.ed[16 * t + 4 * lq]);
            Dd[t] = f32x4_t{ed.x * D[t][0], ed.y * D[t][1], ed.z * D[t][2], ed.w * D[t][3]};
        }
        const float elast = cm.eg[63];
        const uint4 BT[2] = {pack_f16_frag(Dd[0], Dd[1]), pack_f16_frag(Dd[2], Dd[3])};
#pragma unroll
        for (int j = 0; j < NKB; ++j) ST[j] *= elast;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int j = 0; j < NKB; ++j) ST[j] = mfma_f16(KT[j][hf], BT[hf], ST[j]);
    };

    // runs chunks c0 .. of the range and returns how many it computed (fewer than len: it
    // stopped at a matching record, SEG >= 2)
    auto run = [&](long c0, long len, int g) {
        for (int i = 0;; ++i) {
            lds_barrier();  // chunk i's operands are in LDS
            if (range_done(i, len)) return i;
            if constexpr (SEG == 0) {
                if (p.states16) {   // the state entering the chunk, in the fp16 its products take later
                    _Float16* sp = p.states16 + (((cbase + c0 + i) * H + h) * DV + dvw + l16) * DK + 4 * lq;
#pragma unroll
                    for (int j = 0; j < NKB; ++j)
                        *reinterpret_cast<uint2*>(sp + 16 * j) =
                            make_uint2(pack_f16x2(ST[j][0], ST[j][1]), pack_f16x2(ST[j][2], ST[j][3]));
                }
            }
            step(kq[i & 1], mpv[i % 3], c0 + i);
            const int off = i + 1;
            if constexpr (SEG == 1) {   // the walk never compares in segment 0
                if (g > 0 && recorded(off, len)) store_state(seg_state(g, 31 - __builtin_clz(off)));
            }
            if constexpr (CMP) {
                bool same = false;
                if (recorded(off, len)) {
                    const float* rec = seg_state(g, 31 - __builtin_clz(off));
                    unsigned diff = 0;
#pragma unroll
                    for (int j = 0; j < NKB; ++j) {
                        const uint4 r = *reinterpret_cast<const uint4*>(rec + scol + 16 * j);
                        diff |= (r.x ^ __float_as_uint(ST[j][0])) | (r.y ^ __float_as_uint(ST[j][1])) |
                                (r.z ^ __float_as_uint(ST[j][2])) | (r.w ^ __float_as_uint(ST[j][3]));
                    }
                    same = __builtin_amdgcn_ballot_w64(diff != 0) == 0;
                }
                if (lane == 0) match[i & 1][wave] = same ? 1 : 0;
            }
        }
    };

    if constexpr (SEG == 3) {
        // ok: the state SEG = 2 started segment g from was the true one; otherwise ST holds the
        // true state entering segment g
        // segments 1 .. g-1 were fixed by the second pass (the same test as the DMA wave's: both
        // take the same barriers)
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
            if (wave == 0 && lane == 0) reran[seg] = m;
        }
    }
    if constexpr (SEG == 1) {
        store_state(seg_state(seg, p.seg_ncp));
    } else if (SEG != 2 && p.hT) {
        store_state(p.hT + pair * DV * DK);
    }
}

// ----------------------------------------- stage 2, bf16 inputs, chain and output waves
// The chunk step of chunk_propagate_bf16_kernel for 32-column tiles of unsplit chains, with the
// products that only form o taken off the state chain. Per chunk the state depends on the chain
// X = K S^T -> R = V - diag(e^gamma) X -> Delta = Mmat R -> S' = e^{gamma_last} S + Delta^T
// diag(e^{gamma_last - gamma}) K; the output O^T = e^gamma S Q^T + Delta^T P^T needs S and Delta
// but feeds nothing back. Chain wave w (w < 2) owns columns dv0 + 16w .. +15 and steps the
// state; output wave 2 + w forms o for the same columns from the fp16 operands the chain wave
// leaves in LDS: the state entering the chunk (written at the end of the previous chunk, read
// after the chunk's first barrier) and Delta (written before the chunk's second barrier, read
// after it). The DMA wave (wave 4) copies the operands as in chunk_propagate_bf16_kernel. Two
// barriers per chunk; each wave is on its own SIMD, the DMA wave beside chain wave 0.
template <typename TO, int DK, int DV>
__global__ __launch_bounds__(5 * 64) void chunk_propagate_split_kernel(ChunkProblem p) {
    constexpr int DVT = 32, NW = DVT / 16;   // chain waves; output waves NW .. 2NW-1; DMA wave 2NW
    using KQ = KQChunk<DK>;
    using MPV = MPVChunk<DK, DVT>;
    constexpr int NKB = DK / 16, NKS = DK / 32, NTILE = DV / DVT;
    __shared__ KQ kq[2];
    __shared__ MPV mpv[3];
    __shared__ uint4 xs[NW][NKS][64];   // per chain wave: S^T entering the chunk, fp16 right operands
    __shared__ uint4 xd[NW][2][64];     // per chain wave: Delta^T, fp16 left operands

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;

    // (sequence, head) pair and column tile, mapped as in chunk_propagate_bf16_kernel
    const long NP = (long)p.N * H;
    const long bid = blockIdx.x;
    long unit;
    int tile;
    if (NP % 8 == 0) {
        const long x = bid % 8, i = bid / 8;
        tile = (int)(i % NTILE);
        unit = (i / NTILE) * 8 + x;
    } else {
        unit = bid / NTILE;
        tile = (int)(bid % NTILE);
    }
    const int n = p.cu_seqlens ? p.chunk_base[p.N + 1 + (int)(unit / H)] : (int)(unit / H);
    const int h = (int)(unit % H);
    const long pair = (long)n * H + h;
    const int dv0 = tile * DVT;

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    const long cbase = (p.cu_seqlens == nullptr) ? (long)n * p.nc_per_seq : (long)p.chunk_base[n];
    long nchunks = (seos - sbos + kChunk - 1) / kChunk;
    if (cbase + nchunks > p.nc_bound) nchunks = max(0L, p.nc_bound - cbase);
    auto chunk_len = [&](long jc) {
        const long l = seos - (sbos + jc * kChunk);
        return (int)(l < kChunk ? l : kChunk);
    };

    if (wave == 2 * NW) {
        // ------------------------------------------------------------------- DMA wave
        // Issue order: KQ(0) MPV(0) MPV(1), then per chunk c: KQ(c+1) MPV(c+2); at the top of
        // chunk c only MPV(c+1) may still be in flight.
        // Issuing a chunk's 53 copies takes about as long as the chain's work before the second
        // barrier, so Mmat and P of chunk c+2 are issued after it (same order, same counts).
        auto mpv_copy = [&](long jc, auto part) {
            copy_mpv<DK, DV, DVT, true, decltype(part)::value>(mpv[jc % 3], p, sbos + jc * kChunk, chunk_len(jc),
                                                               (cbase + jc) * H + h, h, dv0, lane);
        };
        if (nchunks > 0) {
            copy_kq<DK>(kq[0], p, cbase * H + h, lane);
            mpv_copy(0, std::integral_constant<int, 0>{});
        }
        if (nchunks > 1) mpv_copy(1, std::integral_constant<int, 0>{});
        for (long i = 0;; ++i) {
            if (i + 1 < nchunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kMpvCopies<DK, DVT>));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            lds_barrier_lgkm();   // chunk i's operands are in LDS (fence-free: see chunk_propagate_bf16_kernel)
            if (i == nchunks) return;
            if (i + 1 < nchunks) copy_kq<DK>(kq[(i + 1) & 1], p, (cbase + i + 1) * H + h, lane);
            if (i + 2 < nchunks) mpv_copy(i + 2, std::integral_constant<int, 1>{});
            lds_barrier_lgkm();   // Delta of chunk i written
            if (i + 2 < nchunks) mpv_copy(i + 2, std::integral_constant<int, 2>{});
        }
    }

    if (wave < NW) {
        // ----------------------------------------------------------------- chain waves
        const int dvw = dv0 + 16 * wave;
        f32x4_t ST[NKB];
        const long scol = (dvw + l16) * DK + 4 * lq;   // this lane's offset in a [dv, dk] state
        if (p.h0) {
#pragma unroll
            for (int j = 0; j < NKB; ++j) {
                const float4 x = *reinterpret_cast<const float4*>(p.h0 + pair * DV * DK + scol + 16 * j);
                ST[j] = f32x4_t{x.x, x.y, x.z, x.w};
            }
        } else {
#pragma unroll
            for (int j = 0; j < NKB; ++j) ST[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        uint4 BS[NKS];
        auto put_state = [&]() {   // S^T as fp16 right operands, kept and left for the output wave
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                BS[s] = pack_f16_frag(ST[2 * s], ST[2 * s + 1]);
                xs[wave][s][lane] = BS[s];
            }
        };
        put_state();
        for (long i = 0;; ++i) {
            lds_barrier();   // chunk i's operands (and the output wave's reads of the last state) done
            if (i == nchunks) break;
            const MPV& cm = mpv[i % 3];
            uint4 MF[4][2];
            float4 V4[4], EG4[4];
            // X = K S^T [64 tokens x 16 columns], the K fragments one 32-wide slice ahead; Mmat
            // and the residual terms read during the last slice
            uint4 KF[2][4];
            auto load_k = [&](int s, uint4 (&kf)[4]) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    kf[t] = *reinterpret_cast<const uint4*>(&cm.K[img_off<DK>(16 * t + l16, 32 * s + 4 * lq)]);
            };
            load_k(0, KF[0]);
            f32x4_t X[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) X[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int b = s & 1;
                if (s + 1 < NKS) {
                    load_k(s + 1, KF[b ^ 1]);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        V4[t] = load4_t<uint16_t>(&cm.V[(16 * t + 4 * lq) * DVT + 16 * wave], DVT);
                        EG4[t] = *reinterpret_cast<const float4*>(&cm.eg[16 * t + 4 * lq]);
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf)
                            MF[t][hf] = *reinterpret_cast<const uint4*>(&cm.M[img_off<64>(16 * t + l16, 32 * hf + 4 * lq)]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t) X[t] = mfma_f16(KF[b][t], BS[s], X[t]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // R = V - e^gamma X;  Delta = Mmat R
            f32x4_t R[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                R[t] = f32x4_t{V4[t].x - EG4[t].x * X[t][0], V4[t].y - EG4[t].y * X[t][1],
                               V4[t].z - EG4[t].z * X[t][2], V4[t].w - EG4[t].w * X[t][3]};
            const uint4 BR[2] = {pack_f16_frag(R[0], R[1]), pack_f16_frag(R[2], R[3])};
            f32x4_t D[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) D[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int t = 0; t < 4; ++t) D[t] = mfma_f16(MF[t][hf], BR[hf], D[t]);
            __builtin_amdgcn_sched_barrier(0);
            xd[wave][0][lane] = pack_f16_frag(D[0], D[1]);
            xd[wave][1][lane] = pack_f16_frag(D[2], D[3]);
            // K^T fragments for the state update, read while Delta is handed over
            const int tr = l16 >> 2, tc = 4 * (l16 & 3);
            uint4 KT[NKB][2];
#pragma unroll
            for (int j = 0; j < NKB; ++j) {
                const int c = 16 * j + tc;
                KT[j][0] = lds_frag2_t(&cm.K[img_off<DK>(4 * lq + tr, c)], &cm.K[img_off<DK>(16 + 4 * lq + tr, c)]);
                KT[j][1] = lds_frag2_t(&cm.K[img_off<DK>(32 + 4 * lq + tr, c)], &cm.K[img_off<DK>(48 + 4 * lq + tr, c)]);
            }
            lds_barrier();   // Delta handed over
            // S^T <- e^{gamma_last} S^T + K^T diag(e^{gamma_last - gamma}) Delta
            f32x4_t Dd[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float4 ed = *reinterpret_cast<const float4*>(&cm.ed[16 * t + 4 * lq]);
                Dd[t] = f32x4_t{ed.x * D[t][0], ed.y * D[t][1], ed.z * D[t][2], ed.w * D[t][3]};
            }
            const float elast = cm.eg[63];
            const uint4 BT[2] = {pack_f16_frag(Dd[0], Dd[1]), pack_f16_frag(Dd[2], Dd[3])};
#pragma unroll
            for (int j = 0; j < NKB; ++j) ST[j] *= elast;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int j = 0; j < NKB; ++j) ST[j] = mfma_f16(KT[j][hf], BT[hf], ST[j]);
            put_state();
        }
        if (p.hT) {
#pragma unroll
            for (int j = 0; j < NKB; ++j)
                *reinterpret_cast<float4*>(p.hT + pair * DV * DK + scol + 16 * j) =
                    make_float4(ST[j][0], ST[j][1], ST[j][2], ST[j][3]);
        }
        return;
    }

    // ------------------------------------------------------------------- output waves
    const int w = wave - NW;
    const int dvw = dv0 + 16 * w;
    for (long i = 0;; ++i) {
        lds_barrier();   // chunk i's operands and the state entering it are in LDS
        if (i == nchunks) break;
        const long jc = i;
        const KQ& ck = kq[i & 1];
        const MPV& cm = mpv[i % 3];
        uint4 BS[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) BS[s] = xs[w][s][lane];
        // Y^T = S (diag(e^gamma) Q)^T [16 columns x 64 tokens], Q fragments one slice ahead; P
        // read during the last slice
        uint4 QF[2][4], PF[4][2];
        auto load_q = [&](int s, uint4 (&qf)[4]) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                qf[t] = *reinterpret_cast<const uint4*>(&ck.Q[img_off<DK>(16 * t + l16, 32 * s + 4 * lq)]);
        };
        load_q(0, QF[0]);
        f32x4_t Y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) Y[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int b = s & 1;
            if (s + 1 < NKS) {
                load_q(s + 1, QF[b ^ 1]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        PF[t][hf] = *reinterpret_cast<const uint4*>(&cm.P[img_off<64>(16 * t + l16, 32 * hf + 4 * lq)]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t) Y[t] = mfma_f16(BS[s], QF[b][t], Y[t]);
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();   // Delta of chunk i is in LDS
        const uint4 BD[2] = {xd[w][0][lane], xd[w][1][lane]};
        // O^T = Y^T + Delta^T P^T (lane: token 16t + l16, columns 16 w + 4 lq .. +3), stored
        // through a resource that ends at the chunk's last token row
        f32x4_t O[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) O[t] = Y[t];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int t = 0; t < 4; ++t) O[t] = mfma_f16(BD[hf], PF[t][hf], O[t]);
        if (p.o) {
            constexpr int E = (int)sizeof(TO);
            const long obos = sbos + jc * kChunk;
            const auto orr = make_rsrc(static_cast<TO*>(p.o) + (obos * H + h) * DV + dvw,
                                       (unsigned)(((chunk_len(jc) - 1) * H * DV + 16) * E));
#pragma unroll
            for (int t = 0; t < 4; ++t) buf_store4<TO>(orr, ((16 * t + l16) * H * DV + 4 * lq) * E, O[t]);
        }
    }
}

// -------------------------------------------------------------------- launchers
WorkspaceLayout workspace_layout(int B, int T, int H, int dk, int N, int varlen, int elem_bytes) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    WorkspaceLayout w{};
    w.nc_bound = varlen ? ((long)T + (long)N * (kChunk - 1)) / kChunk
                        : (long)B * (((long)T + kChunk - 1) / kChunk);
    const size_t units = (size_t)w.nc_bound * H;
    w.off_base = 0;
    const size_t base_bytes = varlen ? (size_t)(2 * N + 1) * 4 : 0;   // chunk_base, then the chain order
    w.off_gates = al(base_bytes);
    w.off_m = al(w.off_gates + units * 128 * 4);
    w.off_p = al(w.off_m + units * 4096 * elem_bytes);
    w.total = w.off_p + units * 4096 * elem_bytes;
    if (elem_bytes == 2) {  // fp16 copies of K and of diag(e^gamma) Q
        w.off_k16 = al(w.total);
        w.off_q16 = al(w.off_k16 + units * 64 * dk * 2);
        w.total = w.off_q16 + units * 64 * dk * 2;
    }
    if (w.nc_bound == 0) w.total = al(base_bytes);
    return w;
}

// The bf16 state propagation runs one work-group per (sequence, head, tile of 32 or 64 d_v
// columns), one per CU (its LDS use admits no second). 64-column tiles read the chunk operands
// from LDS once per 64 columns and keep all four matrix cores busy, so they come first; 32-column
// tiles serve problems that have too few 64-column tiles to fill the device but enough 32-column
// ones. Below that the chains are cut into segments (64-column tiles), aiming at kSegTargetGroups
// work-groups on a 256-CU gfx950 part, with segments of at least kSegMinChunks chunks.
constexpr int kSegTargetGroups = 256;
constexpr int kSegMinChunks = 16;
// the one-kernel forward (d_k = d_v = 128) splits down to 8-chunk segments: its fix-up passes
// cost about one chunk's work per segment
constexpr int kFusedMinChunks = 8;

static long tiles_of(int N, int H, int dv, int cols) { return (long)N * H * (dv > cols ? dv / cols : 1); }

// d_v columns per work-group of the bf16 state propagation (without a split)
static int prop_cols(int N, int H, int dv) {
    return tiles_of(N, H, dv, 64) < kSegTargetGroups && tiles_of(N, H, dv, 32) >= kSegTargetGroups ? 32 : 64;
}

SegPlan segment_plan(int T, int H, int dk, int dv, int N, int bf16) {
    SegPlan sp{1, 0, 0, 0};
    const long nmax = ((long)T + kChunk - 1) / kChunk;   // chunks of the longest possible sequence
    if (!bf16 || nmax < 2) return sp;
    const long tiles = tiles_of(N, H, dv, 64);
    long len = 0;
    if (const char* env = std::getenv("GDN_SEGMENT_CHUNKS")) {
        len = std::atol(env);
        if (len <= 0) return sp;
    } else if (fused_wanted(N, H, dk, dv, bf16)) {   // the one-kernel forward: one work-group per pair
        const long pairs = (long)N * H;
        const long g = std::min((long)kSegTargetGroups / pairs, nmax / kFusedMinChunks);
        if (g < 2) return sp;
        len = (nmax + g - 1) / g;
    } else {
        if (prop_cols(N, H, dv) != 64) return sp;
        const long g = std::min((long)kSegTargetGroups / tiles, nmax / kSegMinChunks);
        if (g < 2) return sp;
        len = (nmax + g - 1) / g;
    }
    const long n = (nmax + len - 1) / len;
    if (n < 2 || tiles * n > 0x7fffffffL) return sp;   // grid size
    sp.n = (int)n;
    sp.len = (int)len;
    while ((1L << sp.ncp) < len) ++sp.ncp;   // offsets 1, 2, 4, .. below len
    sp.bytes = (size_t)N * H * n * ((sp.ncp + 2) * dv * dk * sizeof(float)) + (size_t)tiles * n * sizeof(int32_t);
    return sp;
}

template <typename TIn, int DK, bool BWD>
static hipError_t prep_launch(const ChunkProblem& p, hipStream_t s) {
    // persistent grid: as many work-groups as the device holds at once, so that every
    // (chunk, head) unit is taken by an already running work-group
    static std::atomic<int> resident[64];
    const long cap = resident_blocks(chunk_prepare_kernel<TIn, DK, BWD>, 256, resident, 2);
    const long units = p.nc_bound * p.H;
    const long blocks = units < cap ? units : cap;
    return launch(chunk_prepare_kernel<TIn, DK, BWD>, dim3((unsigned)blocks), dim3(256), s, p);
}

hipError_t launch_chunk_base(const ChunkProblem& p, hipStream_t s) {
    if (!p.cu_seqlens) return hipSuccess;
    return launch(chunk_base_kernel, dim3(1), dim3(1024), s, p.cu_seqlens, p.N, p.T, p.chunk_base);
}

template <bool BWD>
static hipError_t prep_dispatch(const ChunkProblem& p, hipStream_t s) {
    if (p.bf16)
        return p.dk == 64 ? prep_launch<uint16_t, 64, BWD>(p, s) : prep_launch<uint16_t, 128, BWD>(p, s);
    return p.dk == 64 ? prep_launch<float, 64, BWD>(p, s) : prep_launch<float, 128, BWD>(p, s);
}

// p.tmat or p.tmat16 set (the backward pass): the BWD instance
hipError_t launch_chunk_prepare(const ChunkProblem& p, hipStream_t s) {
    hipError_t e = launch_chunk_base(p, s);
    if (e == hipSuccess && p.nc_bound > 0)
        e = (p.tmat || p.tmat16) ? prep_dispatch<true>(p, s) : prep_dispatch<false>(p, s);
    return e;
}

// bf16: DVT/16 compute waves and a DMA wave per work-group (OUT = false: the state chain alone,
// unsplit)
template <typename TO, int DK, int DV, int DVT, bool OUT = true>
static hipError_t prop_launch_bf16(const ChunkProblem& p, hipStream_t s) {
    const long blocks = (long)p.N * p.H * (DV / DVT);
    const dim3 block((DVT / 16 + 1) * 64);
    if constexpr (!OUT) return launch(chunk_propagate_bf16_kernel<TO, DK, DV, DVT, 0, false>, dim3((unsigned)blocks), block, s, p);
    if (p.seg_n <= 1) return launch(chunk_propagate_bf16_kernel<TO, DK, DV, DVT, 0>, dim3((unsigned)blocks), block, s, p);
    hipError_t e = launch(chunk_propagate_bf16_kernel<TO, DK, DV, DVT, 1>, dim3((unsigned)(blocks * p.seg_n)), block, s, p);
    if (e == hipSuccess)
        e = launch(chunk_propagate_bf16_kernel<TO, DK, DV, DVT, 2>, dim3((unsigned)(blocks * (p.seg_n - 1))), block, s, p);
    return e != hipSuccess ? e : launch(chunk_propagate_bf16_kernel<TO, DK, DV, DVT, 3>, dim3((unsigned)blocks), block, s, p);
}

// 32-column tiles of unsplit chains: the chain and output waves of chunk_propagate_split_kernel
// (GDN_SPLIT_OUT=0 selects the four-wave chunk_propagate_bf16_kernel instead)
static bool split_out_wanted() {
    const char* env = std::getenv("GDN_SPLIT_OUT");
    return env ? std::atoi(env) != 0 : true;
}

template <typename TIn, typename TO, int DK, int DV, bool OUT = true>
static hipError_t prop_launch(const ChunkProblem& p, hipStream_t s) {
    if constexpr (sizeof(TIn) == 2) {
        if (p.seg_n <= 1 && prop_cols(p.N, p.H, DV) == 32) {
            if constexpr (OUT && DV >= 32) {
                if (split_out_wanted())
                    return launch(chunk_propagate_split_kernel<TO, DK, DV>, dim3((unsigned)((long)p.N * p.H * (DV / 32))),
                                  dim3(5 * 64), s, p);
            }
            return prop_launch_bf16<TO, DK, DV, 32, OUT>(p, s);
        }
        return prop_launch_bf16<TO, DK, DV, (DV < 64 ? DV : 64), OUT>(p, s);
    } else {
        static_assert(OUT, "the fp32 state propagation always writes o");                            // two waves of 16 columns (LDS size)
        constexpr int DVT = 32;
        const long blocks = (long)p.N * p.H * (DV / DVT);
        return launch(chunk_propagate_kernel<TIn, TO, DK, DV, DVT>, dim3((unsigned)blocks),
                      dim3(DVT / 16 * 64), s, p);
    }
}

template <typename TIn, typename TO, bool OUT = true>
static hipError_t prop_dispatch(const ChunkProblem& p, hipStream_t s) {
    if (p.dk == 64)
        return p.dv == 64 ? prop_launch<TIn, TO, 64, 64, OUT>(p, s) : prop_launch<TIn, TO, 64, 128, OUT>(p, s);
    return p.dv == 64 ? prop_launch<TIn, TO, 128, 64, OUT>(p, s) : prop_launch<TIn, TO, 128, 128, OUT>(p, s);
}

// The state recompute of the backward pass for bf16 inputs: the DMA-fed stage 2 on the fp16
// images its stage 1 wrote (p.k16, p.q16, p.mimg16, p.pimg16), keeping the state entering every
// chunk in fp16 (p.states16) and writing no output.
hipError_t launch_chunk_propagate_states16(const ChunkProblem& p, hipStream_t s) {
    ChunkProblem q = p;
    q.seg_n = 1;   // the states of every chunk are wanted: no split
    q.mmat = p.mimg16;
    q.pmat = p.pimg16;
    q.o = nullptr;
    q.hT = nullptr;
    return (long)p.N * p.H > 0 ? prop_dispatch<uint16_t, float, false>(q, s) : hipSuccess;
}

hipError_t launch_chunk_propagate(const ChunkProblem& p, hipStream_t s) {
    if ((long)p.N * p.H == 0) return hipSuccess;
    if (!p.bf16) return prop_dispatch<float, float>(p, s);
    return p.o_bf16 ? prop_dispatch<uint16_t, uint16_t>(p, s) : prop_dispatch<uint16_t, float>(p, s);
}

}  // namespace gdn
