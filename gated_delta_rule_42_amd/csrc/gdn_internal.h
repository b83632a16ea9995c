// Host-side launch descriptors shared by the C ABI layer and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

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
    int32_t* chunk_base;         // [N + 1] (varlen only)
    float* gates;                // [nc_bound, H, 128]: e^gamma (64), e^{gamma_last - gamma} (64)
    void* mmat;                  // [nc_bound, H, 64, 64] operand type (fp16 or fp32)
    void* pmat;                  // [nc_bound, H, 64, 64] operand type
    _Float16* k16;               // [nc_bound, H, 64, dk] fp16 K (bf16 inputs only)
    _Float16* q16;               // [nc_bound, H, 64, dk] fp16 diag(e^gamma) Q (bf16 inputs only)
};

struct WorkspaceLayout {
    size_t off_base, off_gates, off_m, off_p, off_k16, off_q16, total;
    long nc_bound;
};

WorkspaceLayout workspace_layout(int B, int T, int H, int dk, int N, int varlen, int elem_bytes);

hipError_t launch_chunk_prepare(const ChunkProblem& p, hipStream_t s);
hipError_t launch_chunk_propagate(const ChunkProblem& p, hipStream_t s);

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
};

hipError_t launch_decode(const DecodeProblem& p, hipStream_t s);

}  // namespace gdn
