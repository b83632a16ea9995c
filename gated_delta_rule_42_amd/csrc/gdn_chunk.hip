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
//   Nmat  = P Mmat
//   R     = V - diag(e^gamma) K S^T
//   Delta = Mmat R  (= U - W S^T)                                       effective writes
//   O     = diag(e^gamma) Q S^T + Nmat R  (= diag(e^gamma) Q S^T + P Delta)
//   S'    = e^{gamma_last} S + Delta^T diag(e^{gamma_last - gamma}) K
//
// Stage 1 (chunk_prepare_kernel) computes gamma, Mmat and Nmat for every chunk in
// parallel. Stage 2 (chunk_propagate_kernel) walks the chunks of one (sequence, head,
// d_v tile) in order, keeping the fp32 state tile in registers, and writes O.
// Every gate factor is exp of a non-positive difference, masked before the exp.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// ------------------------------------------------------------------ chunk table
// base[n] = number of chunks in sequences 0..n-1 (each sequence is cut into 64-token
// chunks from its own start); base[N] = total. Token ranges are clamped to [0, T] so a
// malformed offset array cannot move any later access out of bounds.
__global__ __launch_bounds__(1024) void chunk_base_kernel(const int32_t* __restrict__ cu, int N,
                                                          int T, int32_t* __restrict__ base) {
    __shared__ int32_t part[1024];
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
}

// Token range of sequence n, clamped to [0, T] (see chunk_base_kernel).
__device__ __forceinline__ void seq_range(const ChunkProblem& p, int n, long& bos, long& eos) {
    if (p.cu_seqlens == nullptr) {
        bos = (long)n * p.T;
        eos = bos + p.T;
    } else {
        const int b0 = min(max(p.cu_seqlens[n], 0), p.T);
        const int b1 = min(max(p.cu_seqlens[n + 1], b0), p.T);
        bos = b0;
        eos = b1;
    }
}

// Global chunk index c -> first token and length; false if c is past the last chunk.
__device__ __forceinline__ bool locate_chunk(const ChunkProblem& p, long c, long& bos, int& len) {
    int n;
    long j;
    if (p.cu_seqlens == nullptr) {
        n = (int)(c / p.nc_per_seq);
        j = c % p.nc_per_seq;
    } else {
        const long total = min((long)p.chunk_base[p.N], p.nc_bound);
        if (c >= total) return false;
        int lo = 0, hi = p.N;  // largest n with base[n] <= c
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.chunk_base[mid] <= c) lo = mid; else hi = mid;
        }
        n = lo;
        j = c - p.chunk_base[n];
    }
    long sb, se;
    seq_range(p, n, sb, se);
    bos = sb + j * kChunk;
    const long l = se - bos;
    len = (int)(l < kChunk ? l : kChunk);
    return len > 0;
}

// ------------------------------------------------------------------- stage 1
template <typename TM, int DK>
struct alignas(16) PrepSmem {
    static constexpr int PK = DK + 16 / (int)sizeof(TM);  // K, Q row pitch (elements)
    static constexpr int PC = 64 + 16 / (int)sizeof(TM);  // P, Mt row pitch
    static constexpr int PF = 68;                          // fp32 A, T row pitch
    union {
        struct { TM K[64 * PK]; TM Q[64 * PK]; } in;
        struct { float A[64 * PF]; float T[64 * PF]; } tri;
    } u;
    TM P[64 * PC];
    TM Mt[64 * PC];
    float gam[64];
    float beta[64];
};

template <typename TIn, int DK>
__global__ __launch_bounds__(256) void chunk_prepare_kernel(ChunkProblem p) {
    using TM = typename Operand<TIn>::type;
    using SM = PrepSmem<TM, DK>;
    constexpr int PK = SM::PK, PC = SM::PC, PF = SM::PF;
    constexpr int EPV = 16 / (int)sizeof(TM);  // elements per 16-byte vector
    constexpr int VPR = DK / EPV;              // vectors per K / Q row
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;
    const int h = (int)(blockIdx.x % H);
    const long c = blockIdx.x / H;
    long bos;
    int len;
    if (!locate_chunk(p, c, bos, len)) return;
    const long widx = c * H + h;

    // -- load K, Q (rows past the chunk end are zero), g, beta; scan g
    const TIn* kp = static_cast<const TIn*>(p.k);
    const TIn* qp = static_cast<const TIn*>(p.q);
#pragma unroll
    for (int it = 0; it < 64 * VPR / 256; ++it) {
        const int vi = tid + 256 * it;
        const int r = vi / VPR, cv = vi % VPR;
        uint4 kv = zero16(), qv = zero16();
        if (r < len) {
            const long off = ((bos + r) * H + h) * DK + cv * EPV;
            kv = to_operand16<TIn>(*reinterpret_cast<const uint4*>(kp + off));
            qv = to_operand16<TIn>(*reinterpret_cast<const uint4*>(qp + off));
        }
        *reinterpret_cast<uint4*>(&sm.u.in.K[r * PK + cv * EPV]) = kv;
        *reinterpret_cast<uint4*>(&sm.u.in.Q[r * PK + cv * EPV]) = qv;
    }
    if (wave == 0) {
        float gg = 0.f, bb = 0.f;
        if (lane < len) {
            const long o = (bos + lane) * H + h;
            gg = p.g[o];
            bb = p.beta[o];
        }
        float x = gg;  // inclusive prefix sum over the 64 positions
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        sm.gam[lane] = x;
        sm.beta[lane] = bb;
        p.gamma[widx * 64 + lane] = x;
    }
    __syncthreads();

    // -- K K^T and Q K^T on MFMA; wave w owns row block w, column blocks <= w
    const int rb = wave;
    f32x4_t G[4], P0[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        G[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        P0[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (cb <= rb) {
            const TM* brow = &sm.u.in.K[(16 * cb + l16) * PK];
            mma_nt<TM, DK>(G[cb], &sm.u.in.K[(16 * rb + l16) * PK], brow);
            mma_nt<TM, DK>(P0[cb], &sm.u.in.Q[(16 * rb + l16) * PK], brow);
        }
    }
    __syncthreads();  // K and Q are dead; their space becomes A and T

    // -- gate the products: A (strictly lower, fp32) and P (lower incl. diagonal)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * rb + 4 * lq + v, i = 16 * cb + l16;
            float a = 0.f, pp = 0.f;
            if (cb <= rb && i <= r) {
                const float e = __expf(sm.gam[r] - sm.gam[i]);
                if (i < r) a = sm.beta[r] * G[cb][v] * e;
                pp = P0[cb][v] * e;
            }
            sm.u.tri.A[r * PF + i] = a;
            sm.P[r * PC + i] = from_f32<TM>(pp);
        }
    }
    __syncthreads();

    // -- T = (I + A)^{-1}: the four 16x16 diagonal blocks by forward substitution, one
    //    column per lane (wave 0) ...
    float* At = sm.u.tri.A;
    float* Tt = sm.u.tri.T;
    if (wave == 0) {
        const int b = lq, jc = l16;
        const float* Ab = At + 16 * b * PF + 16 * b;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == jc) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= Ab[r * PF + i] * x[i];
            x[r] = acc;
        }
        float* Tb = Tt + 16 * b * PF + 16 * b;
#pragma unroll
        for (int r = 0; r < 16; ++r) Tb[r * PF + jc] = x[r];
    }
    __syncthreads();
    // ... then the blocks below the diagonal, one sub-diagonal at a time:
    //    T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj   (fp32 MFMA, 16x16x4)
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int ib = d + wave, jb = ib - d;
            f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            for (int m = jb; m < ib; ++m) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float a = At[(16 * ib + l16) * PF + 16 * m + 4 * s + lq];
                    const float bb = Tt[(16 * m + 4 * s + lq) * PF + 16 * jb + l16];
                    z = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, z, 0, 0, 0);
                }
            }
            // z is in accumulator layout (lane holds rows 4*lq+s of column l16); use it as
            // the right operand with k relabelled to 4*lq + s in step s.
            f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float a = Tt[(16 * ib + l16) * PF + 16 * ib + 4 * lq + s];
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z[s], t, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) Tt[(16 * ib + 4 * lq + v) * PF + 16 * jb + l16] = -t[v];
        }
        __syncthreads();
    }

    // -- Mmat = T diag(beta): to the workspace (row-major) and, transposed, to LDS
    {
        const int r = tid >> 2, c0 = (tid & 3) * 16;
        float mv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int ci = c0 + e;
            const float t = ((ci >> 4) <= (r >> 4)) ? Tt[r * PF + ci] : 0.f;
            mv[e] = t * sm.beta[ci];
            sm.Mt[ci * PC + r] = from_f32<TM>(mv[e]);
        }
        store16<TM>(static_cast<TM*>(p.mmat) + widx * 4096 + r * 64 + c0, mv);
    }
    __syncthreads();

    // -- Nmat = P Mmat, staged through LDS for a coalesced store. P and Mmat are lower
    //    triangular, so the tiles above the diagonal come out exactly zero; computing all
    //    four costs no time (wave 3 needs four anyway) and needs no masking.
    f32x4_t Nacc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        Nacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mma_nt<TM, 64>(Nacc[cb], &sm.P[(16 * rb + l16) * PC], &sm.Mt[(16 * cb + l16) * PC]);
    }
    float* F = sm.u.tri.A;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) F[(16 * rb + 4 * lq + v) * PF + 16 * cb + l16] = Nacc[cb][v];
    __syncthreads();
    {
        const int r = tid >> 2, c0 = (tid & 3) * 16;
        float nv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) nv[e] = F[r * PF + c0 + e];
        store16<TM>(static_cast<TM*>(p.nmat) + widx * 4096 + r * 64 + c0, nv);
    }
}

// ------------------------------------------------------------------- stage 2
template <typename TM, int DK, int DVT>
struct alignas(16) PropSmem {
    static constexpr int PK = DK + 16 / (int)sizeof(TM);
    static constexpr int PC = 64 + 16 / (int)sizeof(TM);
    TM K[64 * PK];
    TM Q[64 * PK];
    TM V[64 * DVT];
    TM M[64 * PC];
    TM Nm[64 * PC];
    TM S[DVT * PK];    // operand copy of the state tile, rows = d_v
    TM Rt[DVT * PC];   // R^T, rows = d_v, columns = tokens
    TM Dt[DVT * PC];   // (diag(e^{gamma_last - gamma}) Delta)^T
    float gam[64];
};

// Global -> register -> LDS staging of one chunk's inputs (K, Q, the V tile, Mmat, Nmat,
// gamma), so that the loads for chunk c+1 are in flight while chunk c is computed.
template <typename TIn, int DK, int DV, int DVT>
struct ChunkStage {
    using TM = typename Operand<TIn>::type;
    static constexpr int EPV = 16 / (int)sizeof(TM);
    static constexpr int VPR_K = DK / EPV, NV_K = 64 * VPR_K / 256;
    static constexpr int VPR_V = DVT / EPV, NV_V = (64 * VPR_V + 255) / 256;
    static constexpr int VPR_M = 64 / EPV, NV_M = 64 * VPR_M / 256;
    using SM = PropSmem<TM, DK, DVT>;
    uint4 rk[NV_K], rq[NV_K], rv[NV_V], rm[NV_M], rn[NV_M];
    float rg;

    __device__ __forceinline__ void load(const ChunkProblem& p, long sbos, long seos, long cbase,
                                         long jc, int h, int dv0, int tid) {
        const int H = p.H;
        const long bos = sbos + jc * kChunk;
        const long lrem = seos - bos;
        const int len = (int)(lrem < kChunk ? lrem : kChunk);
        const long widx = (cbase + jc) * H + h;
        const TIn* kp = static_cast<const TIn*>(p.k);
        const TIn* qp = static_cast<const TIn*>(p.q);
        const TIn* vp = static_cast<const TIn*>(p.v);
#pragma unroll
        for (int it = 0; it < NV_K; ++it) {
            const int vi = tid + 256 * it, r = vi / VPR_K, cv = vi % VPR_K;
            rk[it] = zero16();
            rq[it] = zero16();
            if (r < len) {
                const long off = ((bos + r) * H + h) * DK + cv * EPV;
                rk[it] = *reinterpret_cast<const uint4*>(kp + off);
                rq[it] = *reinterpret_cast<const uint4*>(qp + off);
            }
        }
#pragma unroll
        for (int it = 0; it < NV_V; ++it) {
            const int vi = tid + 256 * it, r = vi / VPR_V, cv = vi % VPR_V;
            rv[it] = zero16();
            if (vi < 64 * VPR_V && r < len)
                rv[it] = *reinterpret_cast<const uint4*>(vp + ((bos + r) * H + h) * DV + dv0 + cv * EPV);
        }
        const uint4* mp = reinterpret_cast<const uint4*>(static_cast<const TM*>(p.mmat) + widx * 4096);
        const uint4* np = reinterpret_cast<const uint4*>(static_cast<const TM*>(p.nmat) + widx * 4096);
#pragma unroll
        for (int it = 0; it < NV_M; ++it) {
            rm[it] = mp[tid + 256 * it];
            rn[it] = np[tid + 256 * it];
        }
        rg = tid < 64 ? p.gamma[widx * 64 + tid] : 0.f;
    }

    __device__ __forceinline__ void store(SM& sm, int tid) const {
        constexpr int PK = SM::PK, PC = SM::PC;
#pragma unroll
        for (int it = 0; it < NV_K; ++it) {
            const int vi = tid + 256 * it, r = vi / VPR_K, cv = vi % VPR_K;
            *reinterpret_cast<uint4*>(&sm.K[r * PK + cv * EPV]) = to_operand16<TIn>(rk[it]);
            *reinterpret_cast<uint4*>(&sm.Q[r * PK + cv * EPV]) = to_operand16<TIn>(rq[it]);
        }
#pragma unroll
        for (int it = 0; it < NV_V; ++it) {
            const int vi = tid + 256 * it;
            if (vi < 64 * VPR_V) *reinterpret_cast<uint4*>(&sm.V[vi * EPV]) = to_operand16<TIn>(rv[it]);
        }
#pragma unroll
        for (int it = 0; it < NV_M; ++it) {
            const int vi = tid + 256 * it, r = vi / VPR_M, cv = vi % VPR_M;
            *reinterpret_cast<uint4*>(&sm.M[r * PC + cv * EPV]) = rm[it];
            *reinterpret_cast<uint4*>(&sm.Nm[r * PC + cv * EPV]) = rn[it];
        }
        if (tid < 64) sm.gam[tid] = rg;
    }
};

template <typename TIn, typename TO, int DK, int DV, int DVT>
__global__ __launch_bounds__(256) void chunk_propagate_kernel(ChunkProblem p) {
    using TM = typename Operand<TIn>::type;
    using SM = PropSmem<TM, DK, DVT>;
    constexpr int PK = SM::PK, PC = SM::PC;
    constexpr int NDB = DVT / 16;                       // d_v blocks in the tile
    constexpr int NKB = DK / 16;                        // d_k blocks
    constexpr int TPW = NDB * NKB / 4;                  // state tiles per wave
    static_assert(TPW >= 1 && ChunkStage<TIn, DK, DV, DVT>::NV_K >= 1, "tile shape");
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;
    constexpr int NTILE = DV / DVT;

    // (sequence, head) pair and d_v tile. When the pair count allows it, the NTILE tiles
    // of one pair get block ids that are equal modulo 8, i.e. land on the same XCD and
    // share its L2 for K, Q and the chunk operators.
    const long P = (long)p.N * H;
    const long bid = blockIdx.x;
    long pair;
    int tile;
    if (P % 8 == 0) {
        const long x = bid % 8, i = bid / 8;
        tile = (int)(i % NTILE);
        pair = (i / NTILE) * 8 + x;
    } else {
        pair = bid / NTILE;
        tile = (int)(bid % NTILE);
    }
    const int n = (int)(pair / H), h = (int)(pair % H);
    const int dv0 = tile * DVT;

    long sbos, seos;
    seq_range(p, n, sbos, seos);
    long cbase = (p.cu_seqlens == nullptr) ? (long)n * p.nc_per_seq : (long)p.chunk_base[n];
    long nchunks = (seos - sbos + kChunk - 1) / kChunk;
    if (cbase + nchunks > p.nc_bound) nchunks = max(0L, p.nc_bound - cbase);

    // -- state tile: registers (fp32, accumulator layout) + operand copy in LDS
    f32x4_t S[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int ti = wave * TPW + u, a = ti / NKB, b = ti % NKB;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 16 * a + 4 * lq + v, col = 16 * b + l16;
            const float x = p.h0 ? p.h0[(pair * DV + dv0 + row) * DK + col] : 0.f;
            S[u][v] = x;
            sm.S[row * PK + col] = from_f32<TM>(x);
        }
    }

    // -- chunk inputs staged through registers one chunk ahead
    ChunkStage<TIn, DK, DV, DVT> stage;
    TO* op = static_cast<TO*>(p.o);
    if (nchunks > 0) stage.load(p, sbos, seos, cbase, 0, h, dv0, tid);
    for (long jc = 0; jc < nchunks; ++jc) {
        __syncthreads();  // all reads of the previous chunk's LDS data are done
        stage.store(sm, tid);
        __syncthreads();
        if (jc + 1 < nchunks) stage.load(p, sbos, seos, cbase, jc + 1, h, dv0, tid);
        const long bos = sbos + jc * kChunk;
        const long lrem = seos - bos;
        const int len = (int)(lrem < kChunk ? lrem : kChunk);
        const float glast = sm.gam[63];

        // step 1-2: X = K S^T, Y = Q S^T (token block = wave); R = V - e^gamma X -> R^T
        f32x4_t Yg[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            f32x4_t x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
            const TM* srow = &sm.S[(16 * db + l16) * PK];
            mma_nt<TM, DK>(x, &sm.K[(16 * wave + l16) * PK], srow);
            mma_nt<TM, DK>(y, &sm.Q[(16 * wave + l16) * PK], srow);
            float r4[4];
            const int col = 16 * db + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * wave + 4 * lq + v;
                const float e = __expf(sm.gam[r]);
                r4[v] = to_f32(sm.V[r * DVT + col]) - e * x[v];
                Yg[db][v] = e * y[v];
            }
            store4<TM>(&sm.Rt[col * PC + 16 * wave + 4 * lq], r4[0], r4[1], r4[2], r4[3]);
        }
        __syncthreads();

        // step 3: Delta = Mmat R, O = e^gamma Q S^T + Nmat R; Delta scaled for the state
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            f32x4_t dl = {0.f, 0.f, 0.f, 0.f}, oi = {0.f, 0.f, 0.f, 0.f};
            const TM* rrow = &sm.Rt[(16 * db + l16) * PC];
            mma_nt<TM, 64>(dl, &sm.M[(16 * wave + l16) * PC], rrow);
            mma_nt<TM, 64>(oi, &sm.Nm[(16 * wave + l16) * PC], rrow);
            float d4[4];
            const int col = 16 * db + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * wave + 4 * lq + v;
                if (r < len) op[((bos + r) * H + h) * DV + dv0 + col] = from_f32<TO>(Yg[db][v] + oi[v]);
                d4[v] = dl[v] * __expf(glast - sm.gam[r]);
            }
            store4<TM>(&sm.Dt[col * PC + 16 * wave + 4 * lq], d4[0], d4[1], d4[2], d4[3]);
        }
        __syncthreads();

        // step 4: S = e^{gamma_last} S + Dt K   (contraction over the chunk's tokens)
        const float eg = __expf(glast);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ti = wave * TPW + u, a = ti / NKB, b = ti % NKB;
            f32x4_t acc = S[u] * eg;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const Frag<TM> fa = load_frag<TM>(&sm.Dt[(16 * a + l16) * PC + 32 * ks + 8 * lq]);
                const Frag<TM> fb = gather_frag<TM>(&sm.K[(32 * ks + 8 * lq) * PK + 16 * b + l16], PK);
                mma_k32(acc, fa, fb);
            }
            S[u] = acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.S[(16 * a + 4 * lq + v) * PK + 16 * b + l16] = from_f32<TM>(acc[v]);
        }
    }

    if (p.hT) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ti = wave * TPW + u, a = ti / NKB, b = ti % NKB;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                p.hT[(pair * DV + dv0 + 16 * a + 4 * lq + v) * DK + 16 * b + l16] = S[u][v];
        }
    }
}

// -------------------------------------------------------------------- launchers
WorkspaceLayout workspace_layout(int B, int T, int H, int N, int varlen, int elem_bytes) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    WorkspaceLayout w{};
    w.nc_bound = varlen ? ((long)T + (long)N * (kChunk - 1)) / kChunk
                        : (long)B * (((long)T + kChunk - 1) / kChunk);
    w.off_base = 0;
    const size_t base_bytes = varlen ? (size_t)(N + 1) * 4 : 0;
    w.off_gamma = al(base_bytes);
    w.off_m = al(w.off_gamma + (size_t)w.nc_bound * H * 64 * 4);
    w.off_n = al(w.off_m + (size_t)w.nc_bound * H * 4096 * elem_bytes);
    w.total = w.off_n + (size_t)w.nc_bound * H * 4096 * elem_bytes;
    if (w.nc_bound == 0) w.total = al(base_bytes);
    return w;
}

template <typename TIn, int DK>
static void prep_launch(const ChunkProblem& p, hipStream_t s) {
    const long blocks = p.nc_bound * p.H;
    hipLaunchKernelGGL((chunk_prepare_kernel<TIn, DK>), dim3((unsigned)blocks), dim3(256), 0, s, p);
}

hipError_t launch_chunk_prepare(const ChunkProblem& p, hipStream_t s) {
    if (p.cu_seqlens)
        hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(1024), 0, s, p.cu_seqlens, p.N, p.T,
                           p.chunk_base);
    if (p.nc_bound > 0) {
        if (p.bf16) {
            if (p.dk == 64) prep_launch<uint16_t, 64>(p, s); else prep_launch<uint16_t, 128>(p, s);
        } else {
            if (p.dk == 64) prep_launch<float, 64>(p, s); else prep_launch<float, 128>(p, s);
        }
    }
    return hipGetLastError();
}

template <typename TIn, typename TO, int DK, int DV>
static void prop_launch(const ChunkProblem& p, hipStream_t s) {
    // d_v rows per work-group; fp32 operands with d_k = 128 use 16 to stay inside 160 KB of LDS
    constexpr int DVT = (sizeof(TIn) == 4 && DK == 128) ? 16 : 32;
    const long blocks = (long)p.N * p.H * (DV / DVT);
    hipLaunchKernelGGL((chunk_propagate_kernel<TIn, TO, DK, DV, DVT>), dim3((unsigned)blocks),
                       dim3(256), 0, s, p);
}

template <typename TIn, typename TO>
static void prop_dispatch(const ChunkProblem& p, hipStream_t s) {
    if (p.dk == 64) {
        if (p.dv == 64) prop_launch<TIn, TO, 64, 64>(p, s); else prop_launch<TIn, TO, 64, 128>(p, s);
    } else {
        if (p.dv == 64) prop_launch<TIn, TO, 128, 64>(p, s); else prop_launch<TIn, TO, 128, 128>(p, s);
    }
}

hipError_t launch_chunk_propagate(const ChunkProblem& p, hipStream_t s) {
    if ((long)p.N * p.H > 0) {
        if (!p.bf16) prop_dispatch<float, float>(p, s);
        else if (p.o_bf16) prop_dispatch<uint16_t, uint16_t>(p, s);
        else prop_dispatch<uint16_t, float>(p, s);
    }
    return hipGetLastError();
}

}  // namespace gdn
