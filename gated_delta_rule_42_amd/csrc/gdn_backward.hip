// Chunked backward pass of the gated delta rule for gfx950: the gradients of a loss with
// respect to q, k, v, g = log alpha, beta and h0, given its gradients dO with respect to the
// outputs and dhT with respect to the final states.
//
// The pages train the layer with the chunkwise algorithm (paper note "Gated Delta Networks:
// Improving Mamba2 with Delta Rule", mechanism paragraph: "parallel training algorithm";
// record "LIT-137", "Key takeaways") but print no gradient formulas. The ones below are the
// adjoint of the chunk equations of the forward pass (gdn_chunk.hip), with E = diag(e^gamma),
// Ed = diag(e^{gamma_last - gamma}), lam = e^{gamma_last}, X = K S^T, R = V - E X,
// Delta = Mmat R, Y = E Q S^T, O = Y + P Delta, S' = lam S + Delta^T Ed K:
//
//   reverse walk over the chunks of a sequence, dS' = gradient reaching the state after the
//   chunk (dhT for the last chunk):
//     Z = K dS'^T,   dDelta = P^T dO + Ed Z,   dR = Mmat^T dDelta  (= dV)
//     dS = lam dS' + (E dO)^T Q - (E dR)^T K      (dS' of the chunk before; dh0 at the start)
//   every chunk independently, given its entering state S and its dS':
//     dP = dO Delta^T (lower incl. diagonal),  dPg = dP * Gamma
//     dMmat = dDelta R^T,  dT = dMmat diag(beta),  dA = strict_lower(-T^T dT T^T)
//     dQ = E dO S + dPg K
//     dK = -E dR S + Ed Delta dS' + dPg^T Q + (dG + dG^T) K,   dG = dA * beta_r * Gamma
//     dbeta_i = sum_r dMmat[r,i] T[r,i] + sum_m dA[i,m] (k_i . k_m) Gamma[i,m]
//     dgamma_r = (dO : Y)_r - (dR : E X)_r - z_r + (dP : P) row r - (dP : P) column r
//                + (dA : A) row r - (dA : A) column r,   z_r = Ed_r (Delta : Z)_r,
//                and the chunk's last row also gets lam (dS' : S) + sum_r z_r
//     dg = reverse cumulative sum of dgamma within the chunk.
// (":" is the sum of an elementwise product over the d_v columns; Gamma[r,i] = e^{gamma_r -
// gamma_i} for i <= r.)
//
// Passes: (1) stage 1 of the forward pass (gate tables, Mmat, P; gram products accumulated
// in fp32) also keeping T, row-major (fp32; for bf16 inputs, read straight from the raw
// inputs: T in fp16, the fp16 LDS images of K, diag(e^gamma) Q, Mmat and P, and the image of
// P's fp16 rounding remainder); (2) stage 2 of the forward pass keeping the state entering
// every chunk instead of writing o (bf16 inputs: in fp16, the precision (4) takes it in); (3) the reverse walk, keeping dS' of every chunk and writing dh0; (4) every (chunk, head)
// on its own. fp32 inputs run (2)-(4) on the fp32 16x16x4 matrix core
// (chunk_propagate_kernel<float>, chunk_bwd_state_kernel, chunk_bwd_grad_kernel). bf16 inputs
// run them on fp16 operands with fp32 accumulation and fp32 state chains: (2) and (3) DMA-fed from
// the images (chunk_propagate_bf16_kernel, chunk_bwd_state16_kernel), (4)
// chunk_bwd_grad16_kernel; the numerics of the forward pass.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_stage2.h"

namespace gdn {

// ------------------------------------------------------- reverse walk (pass 3)
template <int DK, int DVT>
struct alignas(16) BwdStateSmem {
    static constexpr int PK = DK + 4, PC = 68, PV = DVT + 4;
    float K[64 * PK];
    float Q[64 * PK];
    float M[64 * PC];
    float P[64 * PC];
    float dO[64 * PV];   // the work-group's d_v columns
    float eg[64];
    float ed[64];
};

// One work-group per (sequence, head, DVT-column tile); wave w owns d_v columns dv0 + 16w
// .. +15 and holds dS'^T [d_k, 16] as d_k/16 accumulator tiles (lane: dS'[col l16][16j +
// 4 lq + 0..3]), walking the chunks from the last to the first.
template <int DK, int DV, int DVT>
__global__ __launch_bounds__(DVT / 16 * 64) void chunk_bwd_state_kernel(ChunkProblem p, const float* do32,
                                                                         const float* dhT, float* dstates,
                                                                         float* dh0) {
    using SM = BwdStateSmem<DK, DVT>;
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

    f32x4_t dST[NKB];
    const long srow = (pair * DV + dvw + l16) * DK + 4 * lq;
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        if (dhT) {
            const float4 x = *reinterpret_cast<const float4*>(dhT + srow + 16 * j);
            dST[j] = f32x4_t{x.x, x.y, x.z, x.w};
        } else {
            dST[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    const float* kp = static_cast<const float*>(p.k);
    const float* qp = static_cast<const float*>(p.q);
    const float* mp = static_cast<const float*>(p.mmat);
    const float* pp = static_cast<const float*>(p.pmat);

    for (long jc = nchunks - 1; jc >= 0; --jc) {
        const long bos = sbos + jc * 64, widx = (cbase + jc) * H + h;
        const int len = (int)min(64L, seos - bos);
        __syncthreads();  // the previous chunk's LDS data is dead
        for (int i = tid; i < 64 * DK / 4; i += NT) {
            const int r = i / (DK / 4), c = 4 * (i % (DK / 4));
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
            if (r < len) {
                kv = *reinterpret_cast<const float4*>(kp + ((bos + r) * H + h) * DK + c);
                qv = *reinterpret_cast<const float4*>(qp + ((bos + r) * H + h) * DK + c);
            }
            *reinterpret_cast<float4*>(&sm.K[r * PK + c]) = kv;
            *reinterpret_cast<float4*>(&sm.Q[r * PK + c]) = qv;
        }
        for (int i = tid; i < 64 * 16; i += NT) {
            const int r = i / 16, c = 4 * (i % 16);
            *reinterpret_cast<float4*>(&sm.M[r * PC + c]) = *reinterpret_cast<const float4*>(mp + widx * 4096 + r * 64 + c);
            *reinterpret_cast<float4*>(&sm.P[r * PC + c]) = *reinterpret_cast<const float4*>(pp + widx * 4096 + r * 64 + c);
        }
        for (int i = tid; i < 64 * DVT / 4; i += NT) {
            const int r = i / (DVT / 4), c = 4 * (i % (DVT / 4));
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < len) x = *reinterpret_cast<const float4*>(do32 + ((bos + r) * H + h) * DV + dv0 + c);
            *reinterpret_cast<float4*>(&sm.dO[r * PV + c]) = x;
        }
        if (tid < 128) (tid < 64 ? sm.eg : sm.ed)[tid & 63] = p.gates[widx * 128 + tid];
        __syncthreads();

        // dS' of this chunk, for the per-chunk gradients
        float* ds = dstates + (widx * DV + dvw + l16) * DK + 4 * lq;
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            *reinterpret_cast<float4*>(ds + 16 * j) = make_float4(dST[j][0], dST[j][1], dST[j][2], dST[j][3]);

        // Z = K dS'^T (k relabelled to the accumulator rows: step (j, s) takes d_k 16j + 4lq + s)
        f32x4_t Z[4], dD[4], dR[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            Z[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKB; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) Z[t] = mfma4(sm.K[(16 * t + l16) * PK + 16 * j + 4 * lq + s], dST[j][s], Z[t]);
        }
        // dDelta = P^T dO + Ed Z
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            dD[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < 64; k0 += 4)
                dD[t] = mfma4(sm.P[(k0 + lq) * PC + 16 * t + l16], sm.dO[(k0 + lq) * PV + 16 * wave + l16], dD[t]);
#pragma unroll
            for (int m = 0; m < 4; ++m) dD[t][m] += sm.ed[16 * t + 4 * lq + m] * Z[t][m];
        }
        // dR = Mmat^T dDelta
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            dR[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    dR[t] = mfma4(sm.M[(16 * t2 + 4 * lq + s) * PC + 16 * t + l16], dD[t2][s], dR[t]);
        }
        // dS'^T <- lam dS'^T + Q^T (E dO) - K^T (E dR)
        const float lam = sm.eg[63];
        f32x4_t EdR[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int m = 0; m < 4; ++m) EdR[t][m] = -sm.eg[16 * t + 4 * lq + m] * dR[t][m];
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            f32x4_t acc = dST[j] * lam;
#pragma unroll 4
            for (int k0 = 0; k0 < 64; k0 += 4)
                acc = mfma4(sm.Q[(k0 + lq) * PK + 16 * j + l16],
                            sm.eg[k0 + lq] * sm.dO[(k0 + lq) * PV + 16 * wave + l16], acc);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma4(sm.K[(16 * t + 4 * lq + s) * PK + 16 * j + l16], EdR[t][s], acc);
            dST[j] = acc;
        }
    }
    if (dh0) {
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            *reinterpret_cast<float4*>(dh0 + srow + 16 * j) = make_float4(dST[j][0], dST[j][1], dST[j][2], dST[j][3]);
    }
}

// ------------------------------------------------- reverse walk, bf16 inputs (DMA-fed)
// The reverse walk of chunk_bwd_state_kernel on the fp16 matrix core (16x16x32, fp32
// accumulation, the state gradient kept in fp32 and packed to fp16 as an operand). One
// work-group per (sequence, head, DVT-column tile): DVT/16 compute waves (16 columns of dS'
// each) and a DMA wave that copies each chunk's operands into LDS, walking the chunks
// backwards three deep: the fp16 images stage 1 wrote (K, diag(e^gamma) Q, Mmat, P; img_off),
// the gate tables and the raw bf16 dO columns of the work-group (rows past the chunk's end
// read as zeros). The transposed operands (P^T, Mmat^T, Q^T, K^T and dO across tokens) use the
// transposing LDS read at image addresses; k is the chunk's token index throughout. The Q
// image carries diag(e^gamma), so Q^T diag(e^gamma) dO is its transpose times plain dO.
template <int DK, int DVT>
struct alignas(16) BwdWalkChunk {
    _Float16 K[64 * DK];
    _Float16 Q[64 * DK];    // diag(e^gamma) Q
    _Float16 M[64 * 64];    // Mmat
    _Float16 P[64 * 64];
    uint16_t dO[64 * DVT];  // bf16, the work-group's d_v columns
    float gt[128];          // e^gamma, then e^{gamma_last - gamma}
};
template <int DK, int DVT>
constexpr int kWalkCopies = 2 * (64 * DK * 2 / 1024) + 16 + 64 * DVT * 2 / 1024 + 1;

// The DMA wave's copies of one chunk (kWalkCopies instructions, 1 KB blocks).
template <int DK, int DV, int DVT>
__device__ __forceinline__ void walk_copy(BwdWalkChunk<DK, DVT>& dst, const ChunkProblem& p, const uint16_t* dop,
                                          long bos, int len, long widx, int h, int dv0, int lane) {
    constexpr int NB_K = 64 * DK * 2 / 1024, NB_O = 64 * DVT * 2 / 1024, ROW_O = DVT * 2;
    const int H = p.H;
    const unsigned lo = 16u * lane;
    const char* kimg = reinterpret_cast<const char*>(p.k16 + widx * 64 * DK);
    const char* qimg = reinterpret_cast<const char*>(p.q16 + widx * 64 * DK);
    const char* mimg = reinterpret_cast<const char*>(p.mimg16 + widx * 4096);
    const char* pimg = reinterpret_cast<const char*>(p.pimg16 + widx * 4096);
    const auto orr = make_rsrc(dop + (bos * H + h) * DV + dv0, (unsigned)((len - 1) * H * DV + DVT) * 2);
    if (lane < 32) dma16g(reinterpret_cast<const char*>(p.gates + widx * 128), lo, dst.gt);
#pragma unroll
    for (int b = 0; b < NB_O; ++b) {
        const int byte = 1024 * b + 16 * lane, r = byte / ROW_O;
        dma16(orr, reinterpret_cast<const char*>(dst.dO) + 1024 * b, r * H * DV * 2 + 16 * ((byte % ROW_O) >> 4));
    }
#pragma unroll
    for (int b = 0; b < NB_K; ++b) {
        dma16g(kimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.K) + 1024 * b);
        dma16g(qimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.Q) + 1024 * b);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        dma16g(mimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.M) + 1024 * b);
        dma16g(pimg, 1024u * b + lo, reinterpret_cast<const char*>(dst.P) + 1024 * b);
    }
}

// Transposed operand fragment from a [64, W] image: slots 0-3 are column c0 + l16 of rows
// r0 .. r0+3, slots 4-7 of rows r1 .. r1+3 (each lane addresses its own 4-element run).
template <int W>
__device__ __forceinline__ uint4 img_frag_t(const _Float16* img, int r0, int r1, int c0) {
    const int l16 = threadIdx.x & 15, tr = l16 >> 2, tc = 4 * (l16 & 3);
    return lds_frag2_t(&img[img_off<W>(r0 + tr, c0 + tc)], &img[img_off<W>(r1 + tr, c0 + tc)]);
}

template <int DK, int DV, int DVT>
__global__ __launch_bounds__((DVT / 16 + 1) * 64) void chunk_bwd_state16_kernel(ChunkProblem p, const uint16_t* dop,
                                                                                 const float* dhT, float* dstates,
                                                                                 float* dh0) {
    using CH = BwdWalkChunk<DK, DVT>;
    constexpr int NW = DVT / 16, NKB = DK / 16, NKS = DK / 32, NTILE = DV / DVT;
    __shared__ CH ch[3];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;

    // (sequence, head) pair and column tile; with a pair count divisible by 8 the tiles of one
    // pair get block ids equal modulo 8 (same XCD, shared L2 for the pair's operands)
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
    auto chunk_len = [&](long jc) { return (int)min(64L, seos - (sbos + jc * 64)); };

    if (wave == NW) {
        // ------------------------------------------------------------------- DMA wave
        // pass i handles chunk nchunks-1-i; issue order: pass 0, pass 1, then per pass i: pass
        // i+2. Loads complete in issue order, so at the top of pass i only pass i+1 may still be
        // in flight.
        auto copy = [&](long i) {
            const long jc = nchunks - 1 - i;
            walk_copy<DK, DV, DVT>(ch[i % 3], p, dop, sbos + jc * 64, chunk_len(jc), (cbase + jc) * H + h, h, dv0, lane);
        };
        if (nchunks > 0) copy(0);
        if (nchunks > 1) copy(1);
        for (long i = 0; i < nchunks; ++i) {
            if (i + 1 < nchunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kWalkCopies<DK, DVT>));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            // pass i's operands are in LDS; pass i-1's buffers are free. The barrier has no fence:
            // a release fence would make the compiler wait here for every copy in flight (copies
            // write LDS), where the counts above wait for exactly the ones pass i needs
            lds_barrier_lgkm();
            if (i + 2 < nchunks) copy(i + 2);
        }
        return;
    }

    // ------------------------------------------------------------------- compute waves
    // wave w: columns dv0 + 16w .. +15; lane holds dS'[dv0 + 16w + l16][16j + 4lq + 0..3] in dST[j]
    const int dvw = dv0 + 16 * wave;
    f32x4_t dST[NKB];
    const long srow = (pair * DV + dvw + l16) * DK + 4 * lq;
    {
        // dhT through a resource of zero size when there is none (loads read 0)
        const auto hr = make_rsrc(dhT ? dhT + (pair * DV + dvw) * DK : nullptr, dhT ? (unsigned)(16 * DK * 4) : 0u);
#pragma unroll
        for (int j = 0; j < NKB; ++j)
            dST[j] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(hr, (l16 * DK + 4 * lq + 16 * j) * 4, 0, 0));
    }

    for (long i = 0, m3 = 0; i < nchunks; ++i, m3 = (m3 == 2 ? 0 : m3 + 1)) {
        const long jc = nchunks - 1 - i, widx = (cbase + jc) * H + h;
        const CH& cm = ch[m3];
        lds_barrier();  // this pass's operands are in LDS

        float* ds = dstates + (widx * DV + dvw + l16) * DK + 4 * lq;
#pragma unroll
        for (int j = 0; j < NKB; ++j) *reinterpret_cast<f32x4_t*>(ds + 16 * j) = dST[j];

        // Z = K dS'^T
        uint4 BS[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) BS[s] = pack_f16_frag(dST[2 * s], dST[2 * s + 1]);
        f32x4_t Z[4], dD[4], dR[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            Z[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                Z[t] = mfma_f16(*reinterpret_cast<const uint4*>(&cm.K[img_off<DK>(16 * t + l16, 32 * s + 4 * lq)]),
                                BS[s], Z[t]);
        }
        // dO as a right operand (k = token), bf16 -> fp16
        uint4 DF[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint2 a = lds_read_t16(&cm.dO[(32 * hf + 4 * lq) * DVT + 16 * wave], DVT);
            const uint2 b = lds_read_t16(&cm.dO[(32 * hf + 16 + 4 * lq) * DVT + 16 * wave], DVT);
            DF[hf] = to_operand16<uint16_t>(make_uint4(a.x, a.y, b.x, b.y));
        }
        // dDelta = P^T dO + Ed Z;  dR = -E Mmat^T dDelta
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            dD[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                dD[t] = mfma_f16(img_frag_t<64>(cm.P, 32 * hf + 4 * lq, 32 * hf + 16 + 4 * lq, 16 * t), DF[hf], dD[t]);
            const f32x4_t ed = *reinterpret_cast<const f32x4_t*>(&cm.gt[64 + 16 * t + 4 * lq]);
            dD[t] += ed * Z[t];
        }
        const uint4 BD0 = pack_f16_frag(dD[0], dD[1]), BD1 = pack_f16_frag(dD[2], dD[3]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            dR[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dR[t] = mfma_f16(img_frag_t<64>(cm.M, 4 * lq, 16 + 4 * lq, 16 * t), BD0, dR[t]);
            dR[t] = mfma_f16(img_frag_t<64>(cm.M, 32 + 4 * lq, 48 + 4 * lq, 16 * t), BD1, dR[t]);
            const f32x4_t eg = *reinterpret_cast<const f32x4_t*>(&cm.gt[16 * t + 4 * lq]);
            dR[t] *= -eg;
        }
        // dS'^T <- lam dS'^T + (diag(e^gamma) Q)^T dO - K^T (E dR)
        const uint4 BR0 = pack_f16_frag(dR[0], dR[1]), BR1 = pack_f16_frag(dR[2], dR[3]);
        const float lam = cm.gt[63];
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            f32x4_t acc = dST[j] * lam;
            acc = mfma_f16(img_frag_t<DK>(cm.Q, 4 * lq, 16 + 4 * lq, 16 * j), DF[0], acc);
            acc = mfma_f16(img_frag_t<DK>(cm.Q, 32 + 4 * lq, 48 + 4 * lq, 16 * j), DF[1], acc);
            acc = mfma_f16(img_frag_t<DK>(cm.K, 4 * lq, 16 + 4 * lq, 16 * j), BR0, acc);
            acc = mfma_f16(img_frag_t<DK>(cm.K, 32 + 4 * lq, 48 + 4 * lq, 16 * j), BR1, acc);
            dST[j] = acc;
        }
    }
    if (dh0) {
#pragma unroll
        for (int j = 0; j < NKB; ++j) *reinterpret_cast<f32x4_t*>(dh0 + srow + 16 * j) = dST[j];
    }
}

// ------------------------------------------------------ per-chunk gradients (pass 4)
template <int DK>
struct alignas(16) GradSmem {
    static constexpr int PK = DK + 4, PC = 68, PS = DK + 4, PV = 20;
    float K[64 * PK];
    float Q[64 * PK];
    float T[64 * PC];
    float P[64 * PC];          // P, then dPg
    union {
        struct {               // one 16-column d_v slice
            float S[16 * PS];  // rows dv0 .. +15 of the entering state
            float dS[16 * PS]; // the same rows of dS'
            float V[64 * PV];
            float dO[64 * PV];
            float R[64 * PV];
            float D[64 * PV];  // Delta
            float dD[64 * PV]; // dDelta
            float dR[64 * PV];
        } sl;
        struct {
            float X1[64 * PC]; // dT, then dG
            float X2[64 * PC]; // dT T^T
        } cc;
    } u;
    float gam[64], eg[64], ed[64], beta[64];
    // partial sums of dgamma and dbeta, added in a fixed order (results are reproducible)
    float colg[4][64], colb[4][64];   // column terms, per wave
    float rowg[64], rowb[64];         // row terms (each row belongs to one wave)
    float tailw[4];                   // last-row terms, per wave
};

// Sums over the lanes of a wave that share l16 (the four lq groups), or that share lq (the
// sixteen l16 lanes), or over all 64 lanes. Butterflies: every lane ends with the same value,
// added in an order that does not depend on timing.
__device__ __forceinline__ float sum_lq(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float sum_l16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x + __shfl_xor(x, 8);
}

template <typename TO>
__device__ __forceinline__ void store_elem(TO* p, float x) { *p = from_f32<TO>(x); }

// One work-group (4 waves) per (chunk, head); wave w owns token rows 16w .. 16w+15 of every
// row-blocked product. The d_v-dependent terms are accumulated over 16-column slices of d_v.
template <typename TO, int DK, int DV>
__global__ __launch_bounds__(256) void chunk_bwd_grad_kernel(BwdProblem bp) {
    using SM = GradSmem<DK>;
    constexpr int PK = SM::PK, PC = SM::PC, PS = SM::PS, PV = SM::PV, NKB = DK / 16;
    __shared__ SM sm;
    const ChunkProblem& p = bp.f;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;
    const long unit = blockIdx.x, c = unit / H;
    const int h = (int)(unit % H);
    long bos;
    int len;
    if (!locate_chunk(p, c, bos, len)) return;   // uniform over the work-group
    const long widx = c * H + h;
    const float* kp = static_cast<const float*>(p.k);
    const float* qp = static_cast<const float*>(p.q);
    const float* vp = static_cast<const float*>(p.v);
    const float* dop = bp.do32;

    for (int i = tid; i < 64 * DK / 4; i += 256) {
        const int r = i / (DK / 4), cc = 4 * (i % (DK / 4));
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
        if (r < len) {
            kv = *reinterpret_cast<const float4*>(kp + ((bos + r) * H + h) * DK + cc);
            qv = *reinterpret_cast<const float4*>(qp + ((bos + r) * H + h) * DK + cc);
        }
        *reinterpret_cast<float4*>(&sm.K[r * PK + cc]) = kv;
        *reinterpret_cast<float4*>(&sm.Q[r * PK + cc]) = qv;
    }
    for (int i = tid; i < 64 * 16; i += 256) {
        const int r = i / 16, cc = 4 * (i % 16);
        *reinterpret_cast<float4*>(&sm.T[r * PC + cc]) = *reinterpret_cast<const float4*>(p.tmat + widx * 4096 + r * 64 + cc);
        *reinterpret_cast<float4*>(&sm.P[r * PC + cc]) =
            *reinterpret_cast<const float4*>(static_cast<const float*>(p.pmat) + widx * 4096 + r * 64 + cc);
    }
    if (wave == 0) {
        const long o = (bos + lane) * H + h;
        const float gr = lane < len ? p.g[o] : 0.f;
        sm.beta[lane] = lane < len ? p.beta[o] : 0.f;
        sm.gam[lane] = wave_inclusive_sum(gr);
        sm.eg[lane] = p.gates[widx * 128 + lane];
        sm.ed[lane] = p.gates[widx * 128 + 64 + lane];
    }

    const int row = 16 * wave + l16;   // this lane's row as a left operand
    f32x4_t dP[4], dM[4], dQ1[NKB], dK1[NKB];
#pragma unroll
    for (int t = 0; t < 4; ++t) dP[t] = dM[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NKB; ++j) dQ1[j] = dK1[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float gacc[4] = {0.f, 0.f, 0.f, 0.f};   // dgamma of rows 16 wave + 4 lq + m, this lane's column
    float tail = 0.f;                       // lam (dS' : S) + sum z, this thread's share
    auto& sl = sm.u.sl;

    for (int js = 0; js < DV / 16; ++js) {
        const int dv0 = 16 * js;
        __syncthreads();  // the previous slice is dead (first slice: the loads above are done)
        const float lam = sm.eg[63];
        for (int i = tid; i < 16 * DK / 4; i += 256) {
            const int r = i / (DK / 4), cc = 4 * (i % (DK / 4));
            const float4 s = *reinterpret_cast<const float4*>(p.states + (widx * DV + dv0 + r) * DK + cc);
            const float4 d = *reinterpret_cast<const float4*>(bp.dstates + (widx * DV + dv0 + r) * DK + cc);
            *reinterpret_cast<float4*>(&sl.S[r * PS + cc]) = s;
            *reinterpret_cast<float4*>(&sl.dS[r * PS + cc]) = d;
            tail += lam * (s.x * d.x + s.y * d.y + s.z * d.z + s.w * d.w);
        }
        {
            const int r = tid >> 2, cc = 4 * (tid & 3);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f), d = v;
            if (r < len) {
                v = *reinterpret_cast<const float4*>(vp + ((bos + r) * H + h) * DV + dv0 + cc);
                d = *reinterpret_cast<const float4*>(dop + ((bos + r) * H + h) * DV + dv0 + cc);
            }
            *reinterpret_cast<float4*>(&sl.V[r * PV + cc]) = v;
            *reinterpret_cast<float4*>(&sl.dO[r * PV + cc]) = d;
        }
        __syncthreads();

        // X = K S^T, Y = Q S^T, Z = K dS'^T for this wave's rows
        f32x4_t X = {0.f, 0.f, 0.f, 0.f}, Y = X, Z = X;
#pragma unroll 4
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const float ak = sm.K[row * PK + k0 + lq], aq = sm.Q[row * PK + k0 + lq];
            const float bs = sl.S[l16 * PS + k0 + lq], bd = sl.dS[l16 * PS + k0 + lq];
            X = mfma4(ak, bs, X);
            Y = mfma4(aq, bs, Y);
            Z = mfma4(ak, bd, Z);
        }
        float EX[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            EX[m] = sm.eg[r] * X[m];
            sl.R[r * PV + l16] = sl.V[r * PV + l16] - EX[m];
            gacc[m] += sl.dO[r * PV + l16] * sm.eg[r] * Y[m];
        }
        __syncthreads();

        // Delta = T diag(beta) R, dDelta = P^T dO + Ed Z
        f32x4_t Dl = {0.f, 0.f, 0.f, 0.f}, dDl = Dl;
#pragma unroll 4
        for (int k0 = 0; k0 < 64; k0 += 4) {
            const int i = k0 + lq;
            Dl = mfma4(sm.T[row * PC + i], sm.beta[i] * sl.R[i * PV + l16], Dl);
            dDl = mfma4(sm.P[i * PC + row], sl.dO[i * PV + l16], dDl);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            const float z = sm.ed[r] * Dl[m] * Z[m];
            dDl[m] += sm.ed[r] * Z[m];
            gacc[m] -= z;
            tail += z;
            sl.D[r * PV + l16] = Dl[m];
            sl.dD[r * PV + l16] = dDl[m];
        }
        __syncthreads();

        // dR = Mmat^T dDelta (= dV)
        f32x4_t dRl = {0.f, 0.f, 0.f, 0.f};
        const float brow = sm.beta[row];
#pragma unroll 4
        for (int k0 = 0; k0 < 64; k0 += 4) {
            const int r = k0 + lq;
            dRl = mfma4(sm.T[r * PC + row] * brow, sl.dD[r * PV + l16], dRl);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            gacc[m] -= dRl[m] * EX[m];
            sl.dR[r * PV + l16] = dRl[m];
            if (r < len) store_elem<TO>(static_cast<TO*>(bp.dv) + ((bos + r) * H + h) * DV + dv0 + l16, dRl[m]);
        }
        __syncthreads();

        // dP += dO Delta^T, dMmat += dDelta R^T (contraction over the slice's 16 columns)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4) {
                const int v = k0 + lq;
                dP[cb] = mfma4(sl.dO[row * PV + v], sl.D[(16 * cb + l16) * PV + v], dP[cb]);
                dM[cb] = mfma4(sl.dD[row * PV + v], sl.R[(16 * cb + l16) * PV + v], dM[cb]);
            }
        // dQ1 += E dO S, dK1 += -E dR S + Ed Delta dS'
        const float egr = sm.eg[row], edr = sm.ed[row];
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
            const int v = k0 + lq;
            const float a1 = egr * sl.dO[row * PV + v], a2 = -egr * sl.dR[row * PV + v], a3 = edr * sl.D[row * PV + v];
#pragma unroll
            for (int j = 0; j < NKB; ++j) {
                const float bS = sl.S[v * PS + 16 * j + l16], bdS = sl.dS[v * PS + 16 * j + l16];
                dQ1[j] = mfma4(a1, bS, dQ1[j]);
                dK1[j] = mfma4(a2, bS, dK1[j]);
                dK1[j] = mfma4(a3, bdS, dK1[j]);
            }
        }
    }
    __syncthreads();  // slice buffers are dead; their space becomes X1, X2

    // -- dPg (into P) and the P terms of dgamma; dT (into X1) and the Mmat term of dbeta
    float rowacc[4] = {0.f, 0.f, 0.f, 0.f}, dbrow[4] = {0.f, 0.f, 0.f, 0.f};
    float colg[4] = {0.f, 0.f, 0.f, 0.f}, colb[4] = {0.f, 0.f, 0.f, 0.f};   // column 16 cb + l16
    auto& cc = sm.u.cc;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int col = 16 * cb + l16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            float dpg = 0.f;
            if (col <= r) {
                const float x = dP[cb][m] * sm.P[r * PC + col];
                rowacc[m] += x;
                colg[cb] -= x;
                dpg = dP[cb][m] * __expf(sm.gam[r] - sm.gam[col]);
            }
            sm.P[r * PC + col] = dpg;
            colb[cb] += dM[cb][m] * sm.T[r * PC + col];
            cc.X1[r * PC + col] = dM[cb][m] * sm.beta[col];
        }
    }
    __syncthreads();
    // -- X2 = dT T^T
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < 64; k0 += 4)
            acc = mfma4(cc.X1[row * PC + k0 + lq], sm.T[(16 * cb + l16) * PC + k0 + lq], acc);
#pragma unroll
        for (int m = 0; m < 4; ++m) cc.X2[(16 * wave + 4 * lq + m) * PC + 16 * cb + l16] = acc[m];
    }
    __syncthreads();
    // -- dA = strict_lower(-T^T X2); with G = K K^T: the A terms of dbeta and dgamma, dG into X1
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        f32x4_t ta = {0.f, 0.f, 0.f, 0.f}, G = ta;
#pragma unroll 4
        for (int k0 = 0; k0 < 64; k0 += 4)
            ta = mfma4(sm.T[(k0 + lq) * PC + row], cc.X2[(k0 + lq) * PC + 16 * cb + l16], ta);
#pragma unroll 4
        for (int k0 = 0; k0 < DK; k0 += 4)
            G = mfma4(sm.K[row * PK + k0 + lq], sm.K[(16 * cb + l16) * PK + k0 + lq], G);
        const int col = 16 * cb + l16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            float dg = 0.f;
            if (col < r) {
                const float da = -ta[m], gm = __expf(sm.gam[r] - sm.gam[col]);
                const float ag = G[m] * gm;
                dbrow[m] += da * ag;
                const float aa = da * sm.beta[r] * ag;
                rowacc[m] += aa;
                colg[cb] -= aa;
                dg = da * sm.beta[r] * gm;
            }
            cc.X1[r * PC + col] = dg;
        }
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const float g = sum_lq(colg[cb]), b = sum_lq(colb[cb]);
        if (lq == 0) {
            sm.colg[wave][16 * cb + l16] = g;
            sm.colb[wave][16 * cb + l16] = b;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float g = sum_l16(gacc[m] + rowacc[m]), b = sum_l16(dbrow[m]);
        if (l16 == 0) {
            sm.rowg[16 * wave + 4 * lq + m] = g;
            sm.rowb[16 * wave + 4 * lq + m] = b;
        }
    }
    {
        const float t = sum_l16(sum_lq(tail));
        if (lane == 0) sm.tailw[wave] = t;
    }
    __syncthreads();

    // -- dQ = dQ1 + dPg K, dK = dK1 + dPg^T Q + dG K + dG^T K
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        f32x4_t aq = dQ1[j], ak = dK1[j];
        const int col = 16 * j + l16;
#pragma unroll 4
        for (int k0 = 0; k0 < 64; k0 += 4) {
            const int i = k0 + lq;
            const float bK = sm.K[i * PK + col], bQ = sm.Q[i * PK + col];
            aq = mfma4(sm.P[row * PC + i], bK, aq);
            ak = mfma4(sm.P[i * PC + row], bQ, ak);
            ak = mfma4(cc.X1[row * PC + i], bK, ak);
            ak = mfma4(cc.X1[i * PC + row], bK, ak);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            if (r < len) {
                const long o = ((bos + r) * H + h) * DK + col;
                store_elem<TO>(static_cast<TO*>(bp.dq) + o, aq[m]);
                store_elem<TO>(static_cast<TO*>(bp.dk) + o, ak[m]);
            }
        }
    }
    // -- dg = reverse cumulative sum of dgamma; dbeta
    if (wave == 0) {
        const int r = 63 - lane;
        float dgam = sm.rowg[r] + ((sm.colg[0][r] + sm.colg[1][r]) + (sm.colg[2][r] + sm.colg[3][r]));
        if (r == 63) dgam += (sm.tailw[0] + sm.tailw[1]) + (sm.tailw[2] + sm.tailw[3]);
        const float x = wave_inclusive_sum(dgam);
        if (r < len) {
            bp.dg[(bos + r) * H + h] = x;
            bp.dbeta[(bos + r) * H + h] =
                sm.rowb[r] + ((sm.colb[0][r] + sm.colb[1][r]) + (sm.colb[2][r] + sm.colb[3][r]));
        }
    }
}

// ------------------------------------------- per-chunk gradients, bf16 inputs (fp16 operands)
// The products of chunk_bwd_grad_kernel on the fp16 matrix core (16x16x32, fp32 accumulation):
// every operand tile is staged in LDS as fp16 (the raw bf16 inputs exactly, computed values
// rounded once), results accumulate in fp32. The operands whose single rounding would dominate
// the gradients' error (P, the state gradient, beta R, Delta, Ed Delta, dDelta where it forms
// dV, and dPg) are carried as two fp16 tiles, hi = fp16(x) and lo = fp16(x - hi), and their
// products take one extra MFMA per rounded factor (the lo x lo term is dropped): about 22 bits
// of the operand survive instead of 11. k runs in the slot order of fragments packed from two
// accumulator tiles (4lq + 0..3, then 16 + 4lq + 0..3 of each 32-wide k slice): an operand
// stored along k is read as two 8-byte runs (load_frag2), one stored across k with the
// transposing read (load_frag_t). d_v is processed in 32-column slices so that the d_v
// contractions fill whole 32-wide k slices. Eight waves, two per SIMD (the LDS use admits one
// work-group per CU): wave w % 4 owns the 16-row block w % 4 of every product and wave w / 4 one
// half of its output columns (the slice's 16-column tile w / 4, column blocks 2(w/4), 2(w/4)+1 of
// dP, dMmat and the T products, d_k blocks 4(w/4) .. +3 of dQ and dK), so no product is split
// along its contraction; only the row sums of dgamma and dbeta are added across the two halves.
template <int DK>
struct alignas(16) Grad16Smem {
    static constexpr int PK = DK + 8, PT = 72, PS = DK + 8, PV = 40;
    _Float16 K[64 * PK];
    _Float16 Q[64 * PK];
    _Float16 T[64 * PT];
    _Float16 P[64 * PT], Plo[64 * PT];
    union {
        struct {                 // one 32-column d_v slice
            _Float16 S[32 * PS];   // rows of the entering state
            _Float16 dS[32 * PS], dSlo[32 * PS];  // the same rows of dS'
            _Float16 V[64 * PV], dO[64 * PV], EdO[64 * PV], R[64 * PV], BR[64 * PV], BRlo[64 * PV];
            _Float16 D[64 * PV], Dlo[64 * PV], EdD[64 * PV], EdDlo[64 * PV], dD[64 * PV], dDlo[64 * PV];
            _Float16 EdR[64 * PV];
        } sl;
        struct {
            _Float16 X1[64 * PT];  // dT, then dG
            _Float16 X2[64 * PT];  // dT T^T
            _Float16 X3[64 * PT], X3lo[64 * PT];  // dPg
        } cc;
    } u;
    float gam[64], eg[64], ed[64], beta[64];
    float colg[4][64], colb[4][64];   // [row block][column]: column sums of the block's rows
    float rowg[2][64], rowb[2][64];   // [half][row]: row sums over that half's columns
    float tailw[8];
};

template <typename TO, int DK, int DV>
__global__ __launch_bounds__(512) void chunk_bwd_grad16_kernel(BwdProblem bp) {
    using SM = Grad16Smem<DK>;
    constexpr int PK = SM::PK, PT = SM::PT, PS = SM::PS, PV = SM::PV, NKB = DK / 16, NKS = DK / 32;
    __shared__ SM sm;
    const ChunkProblem& p = bp.f;
    // eight waves: wave w % 4 owns row block w % 4 (`wave`), w / 4 (`half`) the half of every
    // product's output columns it forms (see the struct comment)
    const int tid = threadIdx.x, lane = tid & 63, wave = (tid >> 6) & 3, half = tid >> 8;
    const int l16 = lane & 15, lq = lane >> 4;
    const int H = p.H;
    const long unit = blockIdx.x, c = unit / H;
    const int h = (int)(unit % H);
    long bos;
    int len;
    if (!locate_chunk(p, c, bos, len)) return;   // uniform over the work-group
    const long widx = c * H + h;
    const uint16_t* kp = static_cast<const uint16_t*>(bp.k_in);
    const uint16_t* qp = static_cast<const uint16_t*>(bp.q_in);
    const uint16_t* vp = static_cast<const uint16_t*>(bp.v_in);
    const uint16_t* dop = static_cast<const uint16_t*>(bp.do_in);
    auto pack8 = [](float4 a, float4 b) {
        return make_uint4(pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y), pack_f16x2(b.z, b.w));
    };
    // the fp16 residual x - fp16(x) of eight values whose fp16 rounding is `hi`
    auto resid8 = [](float4 a, float4 b, uint4 hi) {
        const f16x8_t h = __builtin_bit_cast(f16x8_t, hi);
        return make_uint4(pack_f16x2(a.x - (float)h[0], a.y - (float)h[1]), pack_f16x2(a.z - (float)h[2], a.w - (float)h[3]),
                          pack_f16x2(b.x - (float)h[4], b.y - (float)h[5]), pack_f16x2(b.z - (float)h[6], b.w - (float)h[7]));
    };
    auto split = [](float x, _Float16* hi, _Float16* lo, int o) {
        const _Float16 h = (_Float16)x;
        hi[o] = h;
        lo[o] = (_Float16)(x - (float)h);
    };

    // The unit's first loads are all issued before any is used (one memory latency instead of
    // one per group): K, Q (rows past the chunk's end read as zeros through resources sized to
    // the valid rows), T and P, the gates and, further below, the first d_v slice.
    constexpr int NKQ = 64 * DK / 8 / 512;
    u32x4_t kin[NKQ], qin[NKQ];
    {
        const unsigned kbytes = (unsigned)((len - 1) * H * DK + DK) * 2;
        const auto kr = make_rsrc(kp + (bos * H + h) * DK, kbytes);
        const auto qr = make_rsrc(qp + (bos * H + h) * DK, kbytes);
#pragma unroll
        for (int it = 0; it < NKQ; ++it) {
            const int i = tid + 512 * it, r = i / (DK / 8), cc = 8 * (i % (DK / 8)), off = (r * H * DK + cc) * 2;
            kin[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
            qin[it] = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
        }
    }
    // T fp16 row-major; P as fp16 hi + lo, two images (piece i: row r, columns c0..+3, c0+16..+19)
    u32x4_t tin[1], phi[1], plo[1];
#pragma unroll
    for (int it = 0; it < 1; ++it) {
        const int i = tid + 512 * it, r = i / 8, cc = 8 * (i % 8);
        tin[it] = *reinterpret_cast<const u32x4_t*>(p.tmat16 + widx * 4096 + r * 64 + cc);
        phi[it] = reinterpret_cast<const u32x4_t*>(p.pimg16 + widx * 4096)[i];
        plo[it] = reinterpret_cast<const u32x4_t*>(p.plo16 + widx * 4096)[i];
    }
    float gin = 0.f, bin = 0.f, egin = 0.f, edin = 0.f;
    if (tid < 64) {
        const unsigned gbytes = (unsigned)(((len - 1) * H + 1) * 4);
        gin = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.g + bos * H + h, gbytes), lane * H * 4, 0, 0));
        bin = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.beta + bos * H + h, gbytes), lane * H * 4, 0, 0));
        egin = p.gates[widx * 128 + lane];
        edin = p.gates[widx * 128 + 64 + lane];
    }

    const int row = 16 * wave + l16;   // this lane's row as a left operand
    // Every operand of every product here is read from LDS, so k runs in its natural order
    // within a fragment (8 consecutive k per lane): a row read along k is one 16-byte read, and a
    // read across k takes the lane's 8 rows as two transposed 4-row blocks.
    auto rowc = [&](const _Float16* t, int pitch, int r, int k0) {
        Frag<_Float16> f;
        f.v = *reinterpret_cast<const uint4*>(&t[r * pitch + k0 + 8 * lq]);
        return f;
    };
    auto colc = [&](const _Float16* t, int pitch, int k0, int c0) {
        return load_frag_t<_Float16>(&t[(k0 + 8 * lq) * pitch + c0], &t[(k0 + 8 * lq + 4) * pitch + c0], pitch);
    };
    f32x4_t dP[2], dM[2], dQ1[NKB / 2], dK1[NKB / 2];   // the wave's column blocks 2 half + cl, d_k blocks NKB/2 half + jl
#pragma unroll
    for (int t = 0; t < 2; ++t) dP[t] = dM[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jl = 0; jl < NKB / 2; ++jl) dQ1[jl] = dK1[jl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float gacc[4] = {0.f, 0.f, 0.f, 0.f};   // dgamma of rows 16 wave + 4 lq + m
    float tail = 0.f;                       // lam (dS' : S) + sum z, this thread's share
    auto& sl = sm.u.sl;

    // One d_v slice's rows of the entering state and of dS', and its V and dO columns, staged in
    // registers: slice js+1 is loaded while slice js is computed. Native vector types (a
    // struct-typed copy would go through memory); every load is issued (past the last slice
    // they reload it), V and dO rows past the chunk's end read as zeros through buffer resources.
    constexpr int NSP = 32 * DK / 8, NSI = (NSP + 511) / 512;   // 16-byte pieces of a slice's rows
    u32x4_t rs[NSI];
    f32x4_t rd[NSI][2];
    u32x4_t rvo;   // V (half 0) or dO (half 1) rows
    const unsigned vrow_bytes = (unsigned)((len - 1) * H * DV + 32) * 2;
    auto load_slice = [&](int js) __attribute__((always_inline)) {
        const int dv0 = 32 * js;
#pragma unroll
        for (int it = 0; it < NSI; ++it) {
            const int i = tid + 512 * it, r = i / (DK / 8), cc = 8 * (i % (DK / 8));
            if (i >= NSP) break;
            const _Float16* sp = p.states16 + (widx * DV + dv0 + r) * DK + cc;
            const float* dp = bp.dstates + (widx * DV + dv0 + r) * DK + cc;
            rs[it] = *reinterpret_cast<const u32x4_t*>(sp);
            rd[it][0] = *reinterpret_cast<const f32x4_t*>(dp);
            rd[it][1] = *reinterpret_cast<const f32x4_t*>(dp + 4);
        }
        const int r = (tid & 255) >> 2, cc = 8 * (tid & 3), off = (r * H * DV + cc) * 2;
        rvo = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc((half ? dop : vp) + (bos * H + h) * DV + dv0, vrow_bytes), off, 0, 0);
    };
    auto f4 = [](f32x4_t x) { return make_float4(x[0], x[1], x[2], x[3]); };
    load_slice(0);
#pragma unroll
    for (int it = 0; it < NKQ; ++it) {
        const int i = tid + 512 * it, r = i / (DK / 8), cc = 8 * (i % (DK / 8));
        *reinterpret_cast<uint4*>(&sm.K[r * PK + cc]) =
            to_operand16<uint16_t>(make_uint4(kin[it][0], kin[it][1], kin[it][2], kin[it][3]));
        *reinterpret_cast<uint4*>(&sm.Q[r * PK + cc]) =
            to_operand16<uint16_t>(make_uint4(qin[it][0], qin[it][1], qin[it][2], qin[it][3]));
    }
#pragma unroll
    for (int it = 0; it < 1; ++it) {
        const int i = tid + 512 * it, r = i / 8, cc = 8 * (i % 8);
        *reinterpret_cast<uint4*>(&sm.T[r * PT + cc]) = make_uint4(tin[it][0], tin[it][1], tin[it][2], tin[it][3]);
        int pr, pc0;
        img_piece<64>(i, pr, pc0);
        *reinterpret_cast<uint2*>(&sm.P[pr * PT + pc0]) = make_uint2(phi[it][0], phi[it][1]);
        *reinterpret_cast<uint2*>(&sm.P[pr * PT + pc0 + 16]) = make_uint2(phi[it][2], phi[it][3]);
        *reinterpret_cast<uint2*>(&sm.Plo[pr * PT + pc0]) = make_uint2(plo[it][0], plo[it][1]);
        *reinterpret_cast<uint2*>(&sm.Plo[pr * PT + pc0 + 16]) = make_uint2(plo[it][2], plo[it][3]);
    }
    if (tid < 64) {
        sm.beta[lane] = bin;
        sm.gam[lane] = wave_inclusive_sum(gin);
        sm.eg[lane] = egin;
        sm.ed[lane] = edin;
    }

    for (int js = 0; js < DV / 32; ++js) {
        const int dv0 = 32 * js;
        __syncthreads();  // the previous slice is dead (first slice: the loads above are done)
        const float lam = sm.eg[63];
#pragma unroll
        for (int it = 0; it < NSI; ++it) {
            const int i = tid + 512 * it, r = i / (DK / 8), cc = 8 * (i % (DK / 8));
            if (i >= NSP) break;
            const uint4 sh = make_uint4(rs[it][0], rs[it][1], rs[it][2], rs[it][3]);
            const f16x8_t s8 = __builtin_bit_cast(f16x8_t, sh);
            const float4 s0 = make_float4((float)s8[0], (float)s8[1], (float)s8[2], (float)s8[3]),
                         s1 = make_float4((float)s8[4], (float)s8[5], (float)s8[6], (float)s8[7]);
            const float4 d0 = f4(rd[it][0]), d1 = f4(rd[it][1]);
            const uint4 dh = pack8(d0, d1);
            *reinterpret_cast<uint4*>(&sl.S[r * PS + cc]) = sh;
            *reinterpret_cast<uint4*>(&sl.dS[r * PS + cc]) = dh;
            *reinterpret_cast<uint4*>(&sl.dSlo[r * PS + cc]) = resid8(d0, d1, dh);
            tail += lam * (s0.x * d0.x + s0.y * d0.y + s0.z * d0.z + s0.w * d0.w +
                           s1.x * d1.x + s1.y * d1.y + s1.z * d1.z + s1.w * d1.w);
        }
        {
            const int r = (tid & 255) >> 2, cc = 8 * (tid & 3);
            const uint4 x16 = to_operand16<uint16_t>(make_uint4(rvo[0], rvo[1], rvo[2], rvo[3]));
            if (half == 0) {
                *reinterpret_cast<uint4*>(&sl.V[r * PV + cc]) = x16;
            } else {
                *reinterpret_cast<uint4*>(&sl.dO[r * PV + cc]) = x16;
                const f16x8_t dh = __builtin_bit_cast(f16x8_t, x16);
                const float e = sm.eg[r];
                *reinterpret_cast<uint4*>(&sl.EdO[r * PV + cc]) =
                    pack8(make_float4(e * (float)dh[0], e * (float)dh[1], e * (float)dh[2], e * (float)dh[3]),
                          make_float4(e * (float)dh[4], e * (float)dh[5], e * (float)dh[6], e * (float)dh[7]));
            }
        }
        __syncthreads();
        load_slice(js + 1 < DV / 32 ? js + 1 : js);
        const auto dvr = make_rsrc(static_cast<TO*>(bp.dv) + (bos * H + h) * DV + dv0,
                                   (unsigned)(((len - 1) * H * DV + 32) * (int)sizeof(TO)));

        // X = K S^T, Y = Q S^T, Z = K dS'^T for this wave's rows and its column tile nt = half of
        // the slice
        f32x4_t X[1], Y[1], Z[1];
        X[0] = Y[0] = Z[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const Frag<_Float16> ak = rowc(sm.K, PK, row, 32 * s), aq = rowc(sm.Q, PK, row, 32 * s);
#pragma unroll
            for (int nt0 = 0; nt0 < 1; ++nt0) {
                const int nt = half;
                const Frag<_Float16> bs = rowc(sl.S, PS, 16 * nt + l16, 32 * s), bd = rowc(sl.dS, PS, 16 * nt + l16, 32 * s);
                mma_k32(X[nt0], ak, bs);
                mma_k32(Y[nt0], aq, bs);
                mma_k32(Z[nt0], ak, bd);
                mma_k32(Z[nt0], ak, rowc(sl.dSlo, PS, 16 * nt + l16, 32 * s));
            }
        }
        float EX[1][4];
#pragma unroll
        for (int nt0 = 0; nt0 < 1; ++nt0)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int nt = half;
                const int r = 16 * wave + 4 * lq + m, v = 16 * nt + l16;
                EX[nt0][m] = sm.eg[r] * X[nt0][m];
                const float rv = (float)sl.V[r * PV + v] - EX[nt0][m];
                sl.R[r * PV + v] = (_Float16)rv;
                split(sm.beta[r] * rv, sl.BR, sl.BRlo, r * PV + v);
                gacc[m] += (float)sl.EdO[r * PV + v] * Y[nt0][m];
            }
        __syncthreads();

        // Delta = T (beta R), dDelta = P^T dO + Ed Z
        f32x4_t Dl[1], dDl[1];
#pragma unroll
        for (int nt0 = 0; nt0 < 1; ++nt0) {
            const int nt = half;
            Dl[nt0] = dDl[nt0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < 64; k0 += 32) {
                const Frag<_Float16> at = rowc(sm.T, PT, row, k0), bo = colc(sl.dO, PV, k0, 16 * nt);
                mma_k32(Dl[nt0], at, colc(sl.BR, PV, k0, 16 * nt));
                mma_k32(Dl[nt0], at, colc(sl.BRlo, PV, k0, 16 * nt));
                mma_k32(dDl[nt0], colc(sm.P, PT, k0, 16 * wave), bo);
                mma_k32(dDl[nt0], colc(sm.Plo, PT, k0, 16 * wave), bo);
            }
        }
#pragma unroll
        for (int nt0 = 0; nt0 < 1; ++nt0)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int nt = half;
                const int r = 16 * wave + 4 * lq + m, v = 16 * nt + l16;
                const float z = sm.ed[r] * Dl[nt0][m] * Z[nt0][m];
                dDl[nt0][m] += sm.ed[r] * Z[nt0][m];
                gacc[m] -= z;
                tail += z;
                split(Dl[nt0][m], sl.D, sl.Dlo, r * PV + v);
                split(sm.ed[r] * Dl[nt0][m], sl.EdD, sl.EdDlo, r * PV + v);
                split(dDl[nt0][m], sl.dD, sl.dDlo, r * PV + v);
            }
        __syncthreads();

        // dR = diag(beta) T^T dDelta (= dV)
#pragma unroll
        for (int nt0 = 0; nt0 < 1; ++nt0) {
            const int nt = half;
            f32x4_t dRl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < 64; k0 += 32) {
                const Frag<_Float16> at = colc(sm.T, PT, k0, 16 * wave);
                mma_k32(dRl, at, colc(sl.dD, PV, k0, 16 * nt));
                mma_k32(dRl, at, colc(sl.dDlo, PV, k0, 16 * nt));
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 16 * wave + 4 * lq + m, v = 16 * nt + l16;
                const float d = sm.beta[r] * dRl[m];
                gacc[m] -= d * EX[nt0][m];
                sl.EdR[r * PV + v] = (_Float16)(-sm.eg[r] * d);
                const int off = (r * H * DV + v) * (int)sizeof(TO);   // rows past the end fall outside dvr
                if constexpr (sizeof(TO) == 2)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(d), dvr, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(d), dvr, off, 0, 0);
            }
        }
        __syncthreads();

        // dP += dO Delta^T, dMmat += dDelta R^T, dQ1 += E dO S, dK1 += -E dR S + Ed Delta dS'
        {
            const Frag<_Float16> ao = rowc(sl.dO, PV, row, 0), ad = rowc(sl.dD, PV, row, 0);
#pragma unroll
            for (int cl = 0; cl < 2; ++cl) {
                const int ct = 2 * half + cl;
                mma_k32(dP[cl], ao, rowc(sl.D, PV, 16 * ct + l16, 0));
                mma_k32(dP[cl], ao, rowc(sl.Dlo, PV, 16 * ct + l16, 0));
                mma_k32(dM[cl], ad, rowc(sl.R, PV, 16 * ct + l16, 0));
            }
            const Frag<_Float16> a1 = rowc(sl.EdO, PV, row, 0), a2 = rowc(sl.EdR, PV, row, 0),
                                 a3 = rowc(sl.EdD, PV, row, 0), a3l = rowc(sl.EdDlo, PV, row, 0);
#pragma unroll
            for (int jl = 0; jl < NKB / 2; ++jl) {
                const int j = half * (NKB / 2) + jl;
                const Frag<_Float16> bS = colc(sl.S, PS, 0, 16 * j), bdS = colc(sl.dS, PS, 0, 16 * j);
                mma_k32(dQ1[jl], a1, bS);
                mma_k32(dK1[jl], a2, bS);
                mma_k32(dK1[jl], a3, bdS);
                mma_k32(dK1[jl], a3l, bdS);
                mma_k32(dK1[jl], a3, colc(sl.dSlo, PS, 0, 16 * j));
            }
        }
    }
    __syncthreads();  // slice buffers are dead; their space becomes X1, X2, X3

    // -- dPg (X3) and the P terms of dgamma; dT (X1) and the Mmat term of dbeta
    float rowacc[4] = {0.f, 0.f, 0.f, 0.f}, dbrow[4] = {0.f, 0.f, 0.f, 0.f};
    float colg[2] = {0.f, 0.f}, colb[2] = {0.f, 0.f};   // column 16 ct + l16, ct = 2 half + cl
    auto& cc = sm.u.cc;
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * half + cl;
        const int col = 16 * ct + l16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            float dpg = 0.f;
            if (col <= r) {
                const float x = dP[cl][m] * ((float)sm.P[r * PT + col] + (float)sm.Plo[r * PT + col]);
                rowacc[m] += x;
                colg[cl] -= x;
                dpg = dP[cl][m] * __expf(sm.gam[r] - sm.gam[col]);
            }
            split(dpg, cc.X3, cc.X3lo, r * PT + col);
            colb[cl] += dM[cl][m] * (float)sm.T[r * PT + col];
            cc.X1[r * PT + col] = (_Float16)(dM[cl][m] * sm.beta[col]);
        }
    }
    __syncthreads();
    // -- X2 = dT T^T
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * half + cl;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += 32) mma_k32(acc, rowc(cc.X1, PT, row, k0), rowc(sm.T, PT, 16 * ct + l16, k0));
#pragma unroll
        for (int m = 0; m < 4; ++m) cc.X2[(16 * wave + 4 * lq + m) * PT + 16 * ct + l16] = (_Float16)acc[m];
    }
    __syncthreads();
    // -- dA = strict_lower(-T^T X2); with G = K K^T: the A terms of dbeta and dgamma, dG into X1
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * half + cl;
        f32x4_t ta = {0.f, 0.f, 0.f, 0.f}, G = ta;
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += 32) mma_k32(ta, colc(sm.T, PT, k0, 16 * wave), colc(cc.X2, PT, k0, 16 * ct));
#pragma unroll
        for (int s = 0; s < NKS; ++s) mma_k32(G, rowc(sm.K, PK, row, 32 * s), rowc(sm.K, PK, 16 * ct + l16, 32 * s));
        const int col = 16 * ct + l16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            float dg = 0.f;
            if (col < r) {
                const float da = -ta[m], gm = __expf(sm.gam[r] - sm.gam[col]);
                const float ag = G[m] * gm;
                dbrow[m] += da * ag;
                const float aa = da * sm.beta[r] * ag;
                rowacc[m] += aa;
                colg[cl] -= aa;
                dg = da * sm.beta[r] * gm;
            }
            cc.X1[r * PT + col] = (_Float16)dg;
        }
    }
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * half + cl;
        const float g = sum_lq(colg[cl]), b = sum_lq(colb[cl]);
        if (lq == 0) {
            sm.colg[wave][16 * ct + l16] = g;
            sm.colb[wave][16 * ct + l16] = b;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float g = sum_l16(gacc[m] + rowacc[m]), b = sum_l16(dbrow[m]);
        if (l16 == 0) {
            sm.rowg[half][16 * wave + 4 * lq + m] = g;
            sm.rowb[half][16 * wave + 4 * lq + m] = b;
        }
    }
    {
        const float t = sum_l16(sum_lq(tail));
        if (lane == 0) sm.tailw[tid >> 6] = t;
    }
    __syncthreads();

    // -- dQ = dQ1 + dPg K, dK = dK1 + dPg^T Q + dG K + dG^T K
#pragma unroll
    for (int jl = 0; jl < NKB / 2; ++jl) {
        const int j = half * (NKB / 2) + jl;
        f32x4_t aq = dQ1[jl], ak = dK1[jl];
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += 32) {
            const Frag<_Float16> bK = colc(sm.K, PK, k0, 16 * j), bQ = colc(sm.Q, PK, k0, 16 * j);
            mma_k32(aq, rowc(cc.X3, PT, row, k0), bK);
            mma_k32(aq, rowc(cc.X3lo, PT, row, k0), bK);
            mma_k32(ak, colc(cc.X3, PT, k0, 16 * wave), bQ);
            mma_k32(ak, colc(cc.X3lo, PT, k0, 16 * wave), bQ);
            mma_k32(ak, rowc(cc.X1, PT, row, k0), bK);
            mma_k32(ak, colc(cc.X1, PT, k0, 16 * wave), bK);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 16 * wave + 4 * lq + m;
            if (r < len) {
                const long o = ((bos + r) * H + h) * DK + 16 * j + l16;
                store_elem<TO>(static_cast<TO*>(bp.dq) + o, aq[m]);
                store_elem<TO>(static_cast<TO*>(bp.dk) + o, ak[m]);
            }
        }
    }
    // -- dg = reverse cumulative sum of dgamma; dbeta
    if (tid < 64) {
        const int r = 63 - lane;
        float dgam = (sm.rowg[0][r] + sm.rowg[1][r]) + ((sm.colg[0][r] + sm.colg[1][r]) + (sm.colg[2][r] + sm.colg[3][r]));
        if (r == 63)
            dgam += ((sm.tailw[0] + sm.tailw[1]) + (sm.tailw[2] + sm.tailw[3])) +
                    ((sm.tailw[4] + sm.tailw[5]) + (sm.tailw[6] + sm.tailw[7]));
        const float x = wave_inclusive_sum(dgam);
        if (r < len) {
            bp.dg[(bos + r) * H + h] = x;
            bp.dbeta[(bos + r) * H + h] =
                (sm.rowb[0][r] + sm.rowb[1][r]) + ((sm.colb[0][r] + sm.colb[1][r]) + (sm.colb[2][r] + sm.colb[3][r]));
        }
    }
}

// -------------------------------------------------------------------- launchers
BwdLayout bwd_workspace_layout(int B, int T, int H, int dk, int dv, int N, int varlen, int bf16) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdLayout w{};
    w.fwd = workspace_layout(B, T, H, dk, N, varlen, 4);
    const size_t units = (size_t)w.fwd.nc_bound * H;
    w.off_t = al(w.fwd.total);
    w.off_states = al(w.off_t + units * 4096 * (bf16 ? 2 : 4));
    w.off_dstates = al(w.off_states + units * dv * dk * (bf16 ? 2 : 4));
    size_t end = w.off_dstates + units * dv * dk * 4;
    if (bf16) {
        w.off_k16 = al(end);
        w.off_q16 = al(w.off_k16 + units * 64 * dk * 2);
        end = w.off_q16 + units * 64 * dk * 2;
    }
    w.total = end;
    return w;
}

template <typename TO, int DK, int DV>
static hipError_t bwd_launch(const BwdProblem& b, hipStream_t s) {
    const ChunkProblem& p = b.f;
    constexpr int DVT = 32;
    const long pairs = (long)p.N * p.H;
    hipError_t e = hipSuccess;
    if (pairs > 0) {
        if (p.mimg16)   // bf16 inputs: stage 1's fp16 images, the raw dO
            e = launch(chunk_bwd_state16_kernel<DK, DV, DVT>, dim3((unsigned)(pairs * (DV / DVT))),
                       dim3((DVT / 16 + 1) * 64), s, p, static_cast<const uint16_t*>(b.do_in), b.dhT,
                       b.dstates, b.dh0);
        else
            e = launch(chunk_bwd_state_kernel<DK, DV, DVT>, dim3((unsigned)(pairs * (DV / DVT))),
                       dim3(DVT / 16 * 64), s, p, b.do32, b.dhT, b.dstates, b.dh0);
    }
    const long units = p.nc_bound * p.H;
    if (e == hipSuccess && units > 0) {
        if (p.mimg16)
            e = launch(chunk_bwd_grad16_kernel<TO, DK, DV>, dim3((unsigned)units), dim3(512), s, b);
        else
            e = launch(chunk_bwd_grad_kernel<TO, DK, DV>, dim3((unsigned)units), dim3(256), s, b);
    }
    return e;
}

template <typename TO>
static hipError_t bwd_dispatch(const BwdProblem& b, hipStream_t s) {
    const int dk = b.f.dk, dv = b.f.dv;
    if (dk == 64)
        return dv == 64 ? bwd_launch<TO, 64, 64>(b, s) : bwd_launch<TO, 64, 128>(b, s);
    return dv == 64 ? bwd_launch<TO, 128, 64>(b, s) : bwd_launch<TO, 128, 128>(b, s);
}

hipError_t launch_chunk_backward(const BwdProblem& b, hipStream_t s) {
    const ChunkProblem& p = b.f;
    // stage 1 again (bf16 inputs: straight from the raw inputs, with T in fp16 row-major and
    // the fp16 images of K, diag(e^gamma) Q, Mmat, P and P's rounding remainder), then the
    // state recompute
    hipError_t e = launch_chunk_prepare(p, s);
    if (e != hipSuccess) return e;
    e = p.mimg16 ? launch_chunk_propagate_states16(p, s)   // bf16 inputs: fp16 operands
                 : launch_chunk_propagate(p, s);
    if (e != hipSuccess) return e;
    return b.grad_bf16 ? bwd_dispatch<uint16_t>(b, s) : bwd_dispatch<float>(b, s);
}

}  // namespace gdn
