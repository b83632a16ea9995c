// Host-side launch descriptors shared by the C ABI layer and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace gdn {

// Kernel launch that reports its own status (not a sticky error left by an earlier HIP call
// of the caller, and without clearing one). The trailing arguments are converted to the
// kernel's parameter types.
template <typename T> struct NoDeduce { using type = T; };
template <typename... KArgs>
inline hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         typename NoDeduce<KArgs>::type... args) {
    void* argv[] = {static_cast<void*>(&args)..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, 0, s);
}

// Work-groups of `kern` (block threads, no dynamic LDS) that the current device holds at
// once, cached per device in `cache` (zero = not yet known). Concurrent first calls may
// both run the query; they store the same value, and the atomics make that race-free.
template <typename K>
inline long resident_blocks(K kern, int block, std::atomic<int> (&cache)[64], int fallback_per_cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::atomic<int>& slot = cache[dev & 63];
    int cap = slot.load(std::memory_order_relaxed);
    if (cap == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            per_cu < 1 || cus < 1)
            per_cu = fallback_per_cu, cus = 256;
        cap = per_cu * cus;
        slot.store(cap, std::memory_order_relaxed);
    }
    return cap;
}

// Resolved problem description for the chunked forward pass.
struct ChunkProblem {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* h0;
    void* o;
    float* hT;
    const int32_t* cu_seqlens;   // NULL: fixed-length rows
    int B, T, H, dk, dv, N;
    int bf16;                    // 1: q, k, v are bf16; 0: fp32
    int o_bf16;                  // 1: o is bf16; 0: fp32
    long nc_bound;               // upper bound on the number of chunks (workspace rows)
    int nc_per_seq;              // chunks per row when cu_seqlens is NULL
    // workspace regions
    int32_t* chunk_base;         // [2N + 1] (varlen only): chunk bases, total, chain order
    float* gates;                // [nc_bound, H, 128]: e^gamma (64), e^{gamma_last - gamma} (64)
    void* mmat;                  // [nc_bound, H, 64, 64] operand type (fp16 or fp32)
    void* pmat;                  // [nc_bound, H, 64, 64] operand type
    _Float16* k16;               // [nc_bound, H, 64, dk] fp16 K (bf16 inputs only)
    _Float16* q16;               // [nc_bound, H, 64, dk] fp16 diag(e^gamma) Q (bf16 inputs only)
    // optional outputs of the fp32 kernels, used by the backward pass (NULL: not written)
    float* tmat;                 // [nc_bound, H, 64, 64] T = (I + A)^{-1} (stage 1)
    _Float16* tmat16;            // the same in fp16 (backward pass, bf16 inputs; tmat NULL)
    float* states;               // [nc_bound, H, dv, dk] state entering each chunk (stage 2)
    _Float16* states16;          // the same in fp16 (backward pass, bf16 inputs; states NULL)
    _Float16* mimg16;            // [nc_bound, H, 64, 64] fp16 LDS images of Mmat and P (stage 1
    _Float16* pimg16;            //   of the backward pass, bf16 inputs; with k16, q16)
    _Float16* plo16;             // [nc_bound, H, 64, 64] image of P - fp16(P), fp16 (the same)
    // channel-wise decay (g is [B,T,H,dk]): chunk operators of the fp32 kernels
    float* khat;                 // [nc_bound, H, 64, dk] K * e^gamma          (fp16 for bf16 inputs)
    float* qhat;                 // [nc_bound, H, 64, dk] Q * e^gamma          (fp16 for bf16 inputs)
    float* kdec;                 // [nc_bound, H, 64, dk] K * e^{gamma_last - gamma} (same)
    float* lam;                  // [nc_bound, H, dk] e^{gamma_last}
    // decoupled gates (replace beta when set): erase [B,T,H,dk], write [B,T,H,dv]
    const float* erase;
    const float* write;
    // long-chain split of the bf16 state propagation (seg_n > 1): the chunks of a sequence are
    // cut into segments of seg_len chunks; segst holds, per (sequence, head) and segment, the
    // states at segment offsets 1, 2, 4, .. < seg_len (seg_ncp of them), the first pass's final
    // state and the second pass's final state, each [dv, dk] fp32; then int32
    // [N*H, max(1, dv/64), seg_n], the chunks the second pass recomputed per segment
    int seg_n, seg_len, seg_ncp;
    float* segst;
};

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
    bos = sb + j * 64;
    const long l = se - bos;
    len = (int)(l < 64 ? l : 64);
    return len > 0;
}

struct WorkspaceLayout {
    size_t off_base, off_gates, off_m, off_p, off_k16, off_q16, total;
    long nc_bound;
};

WorkspaceLayout workspace_layout(int B, int T, int H, int dk, int N, int varlen, int elem_bytes);

// Segment plan of the long-chain split (SegPlan::n == 1: no split) and the bytes of its state
// buffer; GDN_SEGMENT_CHUNKS=L in the environment forces segments of L chunks (0: no split).
struct SegPlan {
    int n, len, ncp;
    size_t bytes;
};
SegPlan segment_plan(int T, int H, int dk, int dv, int N, int bf16);

hipError_t launch_chunk_base(const ChunkProblem& p, hipStream_t s);   // chunk_base (packed only)
// The one-kernel forward (gdn_fused.hip): whether gdn_chunk_fwd takes it for a shape (bf16
// inputs, d_k = d_v = 128, fewer than 64 (sequence, head) pairs; GDN_FUSED=0 or 1 in the
// environment forces the choice for the shapes it supports), and its launch
bool fused_wanted(int N, int H, int dk, int dv, int bf16);
hipError_t launch_chunk_fused(const ChunkProblem& p, hipStream_t s);
hipError_t launch_chunk_prepare(const ChunkProblem& p, hipStream_t s);
hipError_t launch_chunk_propagate(const ChunkProblem& p, hipStream_t s);
hipError_t launch_chunk_propagate_states16(const ChunkProblem& p, hipStream_t s);

// Backward pass. `f` describes the forward problem over the caller's q, k, v with its stage-1
// workspace and the tmat and states regions set (bf16 inputs: tmat16 and states16 instead, and
// mimg16, pimg16, k16, q16); the rest are the backward's own inputs, outputs and regions.
struct BwdProblem {
    ChunkProblem f;
    const void* q_in;            // caller's q, k, v, dO in the caller's dtype
    const void* k_in;
    const void* v_in;
    const void* do_in;
    const float* do32;           // fp32 dO (fp32 inputs only, else NULL)
    const float* dhT;            // NULL: zero
    void* dq;                    // [B,T,H,dk] caller's dtype
    void* dk;
    void* dv;                    // [B,T,H,dv] caller's dtype
    float* dg;                   // [B,T,H]
    float* dbeta;                // [B,T,H]
    float* dh0;                  // [N,H,dv,dk] or NULL
    float* dstates;              // [nc_bound, H, dv, dk] gradient leaving each chunk
    int grad_bf16;               // 1: dq, dk, dv are bf16; 0: fp32
};

struct BwdLayout {
    WorkspaceLayout fwd;         // stage-1 regions (fp32 operands)
    size_t off_t, off_states, off_dstates, off_k16, off_q16, total;
};

BwdLayout bwd_workspace_layout(int B, int T, int H, int dk, int dv, int N, int varlen, int bf16);
hipError_t launch_chunk_backward(const BwdProblem& p, hipStream_t s);

// Channel-wise decay: workspace layout and the two stages (chunk operators, propagation).
struct KdaLayout {
    size_t off_base, off_m, off_p, off_kh, off_qh, off_kd, off_lam, total;
    long nc_bound;
};
KdaLayout kda_workspace_layout(int B, int T, int H, int dk, int N, int varlen, int elem);
hipError_t launch_kda_chunk_fwd(const ChunkProblem& p, hipStream_t s);

struct DecodeProblem {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* o;
    int N, H, dk, dv;
    int bf16;     // q, k, v are bf16 (else fp32)
    int o_bf16;   // o is bf16 (else fp32)
    int channel_gate;   // g is [N, H, dk] (one decay per key channel), else [N, H]
    const float* erase;  // decoupled gates (channel_gate only): [N, H, dk] and [N, H, dv];
    const float* write;  // NULL: beta
};

hipError_t launch_decode(const DecodeProblem& p, hipStream_t s);

// gdn_chunk_fwd's host-side argument checks, leaving out the workspace; returns a gdn_status.
int chunk_fwd_check(const void* q, const void* k, const void* v, const float* g_log_alpha, const float* beta,
                    const float* h0, const void* o, const float* hT, const int32_t* cu_seqlens, int chunk,
                    int B, int T, int H, int dk, int dv, int N, int dtype, int o_dtype);

// gdn_chunk_fwd (argument checks, optional GDN_CHECK offsets check, both stages) on the given
// workspace; returns a gdn_status.
int chunk_fwd(const void* q, const void* k, const void* v, const float* g_log_alpha, const float* beta,
              const float* h0, void* o, float* hT, const int32_t* cu_seqlens, int chunk, int B, int T,
              int H, int dk, int dv, int N, int dtype, int o_dtype, void* workspace,
              size_t workspace_bytes, void* stream);

}  // namespace gdn
