// C ABI of libgdn.so (declared in include/gdn.h): argument checks, workspace layout and
// kernel dispatch. Every check runs before any HIP call, so a rejected call launches
// nothing and touches no device state.
#include "gdn.h"
#include "gdn_internal.h"

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#define GDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Size checks shared by the chunked entry points and their workspace queries (after the dtype,
// chunk and head-dimension checks): B, H >= 1, T >= 0, H <= 32768 (one chunk of one head spans
// 64 token rows of H heads, addressed with 32-bit byte offsets inside the kernels), N = B
// without packed sequences and B = 1, N >= 1 with them, at most 2^40 elements in any token
// tensor and at most 2^30 (sequence, head) pairs. Each product is formed only once its factors
// are known to keep it inside 64 bits.
int shape_check(int B, int T, int H, int dk, int dv, int N, bool varlen) {
    if (B < 1 || H < 1 || H > 32768 || T < 0) return GDN_ERR_SHAPE;
    if (varlen ? (B != 1 || N < 1) : (N != B)) return GDN_ERR_SHAPE;
    const long long tokens = (long long)B * T;   // < 2^62
    if (tokens > (1LL << 40) || tokens * H * (dk > dv ? dk : dv) > (1LL << 40)) return GDN_ERR_SHAPE;
    if ((long long)N * H > (1LL << 30)) return GDN_ERR_SHAPE;
    return GDN_OK;
}

// The forward workspace: the stage-1 regions, then the state records of the long-chain split
struct FwdLayout {
    gdn::WorkspaceLayout w;
    gdn::SegPlan seg;
    size_t off_seg, total;
};
FwdLayout fwd_layout(int B, int T, int H, int dk, int dv, int N, int varlen, int bf16) {
    FwdLayout f;
    f.w = gdn::workspace_layout(B, T, H, dk, N, varlen, bf16 ? 2 : 4);
    f.seg = gdn::segment_plan(T, H, dk, dv, N, bf16);
    f.off_seg = (f.w.total + 255) & ~(size_t)255;
    f.total = f.seg.n > 1 ? f.off_seg + f.seg.bytes : f.w.total;
    return f;
}

// GDN_CHECK=1 in the environment: copy cu_seqlens to the host (this synchronises `stream`) and
// reject offsets that break 0 = cu[0] <= cu[1] <= ... <= cu[N] = T. A debugging aid: without it
// the offsets are a precondition that the kernels only clamp into [0, T].
int debug_check_offsets(const int32_t* cu, int N, int T, hipStream_t s) {
    const char* env = std::getenv("GDN_CHECK");
    if (!cu || !env || std::strcmp(env, "1") != 0) return GDN_OK;
    std::vector<int32_t> h((size_t)N + 1);
    if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return GDN_ERR_HIP;
    if (h[0] != 0 || h[(size_t)N] != T) return GDN_ERR_SHAPE;
    for (int i = 0; i < N; ++i)
        if (h[(size_t)i + 1] < h[(size_t)i]) return GDN_ERR_SHAPE;
    return GDN_OK;
}

// Shared checks of the chunked forward entry points. `need` flags: 1 = q,k,g,beta;
// 2 = v,o. Fills the problem description on success.
int check_chunk(const void* q, const void* k, const void* v, const float* g, const float* beta,
                const float* h0, const void* o, const float* hT, const int32_t* cu, int chunk,
                int B, int T, int H, int dk, int dv, int N, int dtype, int o_dtype,
                const void* ws, size_t ws_bytes, int need, gdn::ChunkProblem* p) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (o_dtype != GDN_F32 && !(o_dtype == GDN_BF16 && dtype == GDN_BF16)) return GDN_ERR_DTYPE;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    const int sc = shape_check(B, T, H, dk, dv, N, cu != nullptr);
    if (sc != GDN_OK) return sc;
    const long long tokens = (long long)B * T;
    if (tokens > 0) {
        if ((need & 1) && (!q || !k || !g || !beta)) return GDN_ERR_NULL;
        if ((need & 2) && (!q || !k || !v || !o)) return GDN_ERR_NULL;
    }
    const void* al16[] = {q, k, v, o, h0, hT};
    for (const void* x : al16)
        if (x && !aligned(x, 16)) return GDN_ERR_ALIGN;
    const void* al4[] = {g, beta, cu};
    for (const void* x : al4)
        if (x && !aligned(x, 4)) return GDN_ERR_ALIGN;
    const FwdLayout f = fwd_layout(B, T, H, dk, dv, N, cu != nullptr, dtype == GDN_BF16);
    const gdn::WorkspaceLayout& w = f.w;
    if (w.nc_bound * H > 0x7fffffffL) return GDN_ERR_SHAPE;
    if (f.total > 0 && (!ws || ws_bytes < f.total)) return GDN_ERR_WORKSPACE;
    if (ws && !aligned(ws, 256)) return GDN_ERR_ALIGN;

    gdn::ChunkProblem& P = *p;
    P.q = q; P.k = k; P.v = v; P.g = g; P.beta = beta; P.h0 = h0;
    P.o = const_cast<void*>(o); P.hT = const_cast<float*>(hT); P.cu_seqlens = cu;
    P.B = B; P.T = T; P.H = H; P.dk = dk; P.dv = dv; P.N = N;
    P.bf16 = dtype == GDN_BF16;
    P.o_bf16 = o_dtype == GDN_BF16;
    P.nc_bound = w.nc_bound;
    P.nc_per_seq = (T + 63) / 64;
    char* base = static_cast<char*>(const_cast<void*>(ws));
    P.chunk_base = cu ? reinterpret_cast<int32_t*>(base + w.off_base) : nullptr;
    P.gates = w.nc_bound ? reinterpret_cast<float*>(base + w.off_gates) : nullptr;
    P.mmat = w.nc_bound ? base + w.off_m : nullptr;
    P.pmat = w.nc_bound ? base + w.off_p : nullptr;
    P.k16 = (w.nc_bound && P.bf16) ? reinterpret_cast<_Float16*>(base + w.off_k16) : nullptr;
    P.q16 = (w.nc_bound && P.bf16) ? reinterpret_cast<_Float16*>(base + w.off_q16) : nullptr;
    P.seg_n = f.seg.n;
    P.seg_len = f.seg.len;
    P.seg_ncp = f.seg.ncp;
    P.segst = f.seg.n > 1 ? reinterpret_cast<float*>(base + f.off_seg) : nullptr;
    return GDN_OK;
}

}  // namespace

GDN_EXPORT int gdn_version(void) { return 100; }

GDN_EXPORT const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "a size is out of range or inconsistent";
        case GDN_ERR_DTYPE: return "unknown dtype code";
        case GDN_ERR_ALIGN: return "a pointer is misaligned (q/k/v/o/states 16 B, gates 4 B, workspace 256 B)";
        case GDN_ERR_UNSUPPORTED: return "unsupported chunk size or head dimension (chunk 64; d_k, d_v in {64, 128})";
        case GDN_ERR_WORKSPACE: return "workspace missing or smaller than gdn_chunk_fwd_workspace_bytes()";
        case GDN_ERR_HIP: return "a HIP launch failed";
        default: return "unknown status";
    }
}

GDN_EXPORT size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                                int varlen, int chunk, int dtype) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return 0;
    if (chunk != 64 || !head_dim_ok(dk) || !head_dim_ok(dv)) return 0;
    if (shape_check(B, T, H, dk, dv, N, varlen != 0) != GDN_OK) return 0;
    return fwd_layout(B, T, H, dk, dv, N, varlen != 0, dtype == GDN_BF16).total;
}

GDN_EXPORT int gdn_chunk_prepare(const void* q, const void* k, const float* g, const float* beta,
                                 const int32_t* cu_seqlens, int chunk, int B, int T, int H, int dk,
                                 int dv, int N, int dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    gdn::ChunkProblem p{};
    int st = check_chunk(q, k, nullptr, g, beta, nullptr, nullptr, nullptr, cu_seqlens, chunk, B, T,
                         H, dk, dv, N, dtype, GDN_F32, workspace, workspace_bytes, 1, &p);
    if (st != GDN_OK) return st;
    st = debug_check_offsets(cu_seqlens, N, T, static_cast<hipStream_t>(stream));
    if (st != GDN_OK) return st;
    return gdn::launch_chunk_prepare(p, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK
                                                                                      : GDN_ERR_HIP;
}

GDN_EXPORT int gdn_chunk_propagate(const void* q, const void* k, const void* v, const float* h0,
                                   void* o, float* hT, const int32_t* cu_seqlens, int chunk, int B,
                                   int T, int H, int dk, int dv, int N, int dtype, int o_dtype,
                                   const void* workspace, size_t workspace_bytes, void* stream) {
    gdn::ChunkProblem p{};
    int st = check_chunk(q, k, v, nullptr, nullptr, h0, o, hT, cu_seqlens, chunk, B, T, H, dk, dv,
                         N, dtype, o_dtype, workspace, workspace_bytes, 2, &p);
    if (st != GDN_OK) return st;
    st = debug_check_offsets(cu_seqlens, N, T, static_cast<hipStream_t>(stream));
    if (st != GDN_OK) return st;
    return gdn::launch_chunk_propagate(p, static_cast<hipStream_t>(stream)) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

namespace gdn {
// gdn_chunk_fwd's argument checks (host only, no HIP call) for a caller that will supply a
// workspace of gdn_chunk_fwd_workspace_bytes(...) bytes itself: GDN_OK or the status
// gdn_chunk_fwd would return for any argument other than the workspace.
int chunk_fwd_check(const void* q, const void* k, const void* v, const float* g_log_alpha, const float* beta,
                    const float* h0, const void* o, const float* hT, const int32_t* cu_seqlens, int chunk,
                    int B, int T, int H, int dk, int dv, int N, int dtype, int o_dtype) {
    gdn::ChunkProblem p{};
    const int st = check_chunk(q, k, v, g_log_alpha, beta, h0, o, hT, cu_seqlens, chunk, B, T, H, dk, dv, N,
                               dtype, o_dtype, nullptr, 0, 3, &p);
    return st == GDN_ERR_WORKSPACE ? GDN_OK : st;
}

// gdn_chunk_fwd with its arguments as given (also serves entry points that supply their own
// workspace)
int chunk_fwd(const void* q, const void* k, const void* v, const float* g_log_alpha, const float* beta,
              const float* h0, void* o, float* hT, const int32_t* cu_seqlens, int chunk, int B, int T,
              int H, int dk, int dv, int N, int dtype, int o_dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
    gdn::ChunkProblem p{};
    int st = check_chunk(q, k, v, g_log_alpha, beta, h0, o, hT, cu_seqlens, chunk, B, T, H, dk, dv,
                         N, dtype, o_dtype, workspace, workspace_bytes, 3, &p);
    if (st != GDN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_offsets(cu_seqlens, N, T, s);
    if (st != GDN_OK) return st;
    if (gdn::fused_wanted(p.N, p.H, p.dk, p.dv, p.bf16))
        return gdn::launch_chunk_fused(p, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    if (gdn::launch_chunk_prepare(p, s) != hipSuccess) return GDN_ERR_HIP;
    if (gdn::launch_chunk_propagate(p, s) != hipSuccess) return GDN_ERR_HIP;
    return GDN_OK;
}
}  // namespace gdn

GDN_EXPORT int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g_log_alpha,
                             const float* beta, const float* h0, void* o, float* hT,
                             const int32_t* cu_seqlens, int chunk, int B, int T, int H, int dk,
                             int dv, int N, int dtype, int o_dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return gdn::chunk_fwd(q, k, v, g_log_alpha, beta, h0, o, hT, cu_seqlens, chunk, B, T, H, dk, dv, N,
                          dtype, o_dtype, workspace, workspace_bytes, stream);
}

GDN_EXPORT int gdn_decode_step(const void* q, const void* k, const void* v, const float* g_log_alpha,
                               const float* beta, float* state, void* o, int N, int H, int dk,
                               int dv, int dtype, int o_dtype, void* stream) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (o_dtype != GDN_F32 && o_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    if (N < 1 || H < 1 || (long long)N * H > 0x7fffffffLL) return GDN_ERR_SHAPE;
    if (!q || !k || !v || !g_log_alpha || !beta || !state || !o) return GDN_ERR_NULL;
    const void* al16[] = {q, k, v, o, state};
    for (const void* x : al16)
        if (!aligned(x, 16)) return GDN_ERR_ALIGN;
    if (!aligned(g_log_alpha, 4) || !aligned(beta, 4)) return GDN_ERR_ALIGN;
    gdn::DecodeProblem p{q,  k, v,  g_log_alpha, beta,           state,
                         o,  N, H,  dk,          dv,   dtype == GDN_BF16, o_dtype == GDN_BF16};
    return gdn::launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK
                                                                                : GDN_ERR_HIP;
}

GDN_EXPORT size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                                int varlen, int chunk, int dtype) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return 0;
    if (chunk != 64 || !head_dim_ok(dk) || !head_dim_ok(dv)) return 0;
    if (shape_check(B, T, H, dk, dv, N, varlen != 0) != GDN_OK) return 0;
    return gdn::bwd_workspace_layout(B, T, H, dk, dv, N, varlen != 0, dtype == GDN_BF16).total;
}

GDN_EXPORT int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g_log_alpha,
                             const float* beta, const float* h0, const void* d_o, const float* dhT,
                             void* dq, void* dk_out, void* dv_out, float* dg, float* dbeta, float* dh0,
                             const int32_t* cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                             int N, int dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (grad_dtype != GDN_F32 && !(grad_dtype == GDN_BF16 && dtype == GDN_BF16)) return GDN_ERR_DTYPE;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    const int sc = shape_check(B, T, H, dk, dv, N, cu_seqlens != nullptr);
    if (sc != GDN_OK) return sc;
    const long long tokens = (long long)B * T;
    if (tokens > 0 && (!q || !k || !v || !g_log_alpha || !beta || !d_o || !dq || !dk_out || !dv_out ||
                       !dg || !dbeta))
        return GDN_ERR_NULL;
    const void* al16[] = {q, k, v, d_o, dq, dk_out, dv_out, h0, dhT, dh0};
    for (const void* x : al16)
        if (x && !aligned(x, 16)) return GDN_ERR_ALIGN;
    const void* al4[] = {g_log_alpha, beta, dg, dbeta, cu_seqlens};
    for (const void* x : al4)
        if (x && !aligned(x, 4)) return GDN_ERR_ALIGN;
    const int bf16 = dtype == GDN_BF16;
    const gdn::BwdLayout w = gdn::bwd_workspace_layout(B, T, H, dk, dv, N, cu_seqlens != nullptr, bf16);
    if (w.fwd.nc_bound * H > 0x7fffffffL) return GDN_ERR_SHAPE;
    if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return GDN_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 256)) return GDN_ERR_ALIGN;

    char* base = static_cast<char*>(workspace);
    gdn::BwdProblem b{};
    gdn::ChunkProblem& P = b.f;
    b.q_in = q; b.k_in = k; b.v_in = v; b.do_in = d_o;
    P.q = q;
    P.k = k;
    P.v = v;
    b.do32 = bf16 ? nullptr : static_cast<const float*>(d_o);
    P.g = g_log_alpha; P.beta = beta; P.h0 = h0; P.o = nullptr; P.hT = nullptr;
    P.cu_seqlens = cu_seqlens;
    P.B = B; P.T = T; P.H = H; P.dk = dk; P.dv = dv; P.N = N;
    P.bf16 = bf16; P.o_bf16 = 0;
    P.nc_bound = w.fwd.nc_bound;
    P.nc_per_seq = (T + 63) / 64;
    const bool any = w.fwd.nc_bound > 0;
    P.chunk_base = cu_seqlens ? reinterpret_cast<int32_t*>(base + w.fwd.off_base) : nullptr;
    P.gates = any ? reinterpret_cast<float*>(base + w.fwd.off_gates) : nullptr;
    P.mmat = any ? base + w.fwd.off_m : nullptr;
    P.pmat = any ? base + w.fwd.off_p : nullptr;
    P.tmat = (any && !bf16) ? reinterpret_cast<float*>(base + w.off_t) : nullptr;
    P.tmat16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.off_t) : nullptr;
    P.states = (any && !bf16) ? reinterpret_cast<float*>(base + w.off_states) : nullptr;
    P.states16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.off_states) : nullptr;
    // bf16: the fp32 Mmat region (not written) holds the fp16 images of Mmat, then of P
    P.mimg16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.fwd.off_m) : nullptr;
    P.pimg16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.fwd.off_m) + w.fwd.nc_bound * H * 4096 : nullptr;
    // bf16: the fp32 P region (not written) holds the image of P's fp16 rounding remainder
    P.plo16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.fwd.off_p) : nullptr;
    P.k16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.off_k16) : nullptr;
    P.q16 = (any && bf16) ? reinterpret_cast<_Float16*>(base + w.off_q16) : nullptr;
    b.dstates = any ? reinterpret_cast<float*>(base + w.off_dstates) : nullptr;
    b.dhT = dhT;
    b.dq = dq; b.dk = dk_out; b.dv = dv_out; b.dg = dg; b.dbeta = dbeta; b.dh0 = dh0;
    b.grad_bf16 = grad_dtype == GDN_BF16;
    const int chk = debug_check_offsets(cu_seqlens, N, T, static_cast<hipStream_t>(stream));
    if (chk != GDN_OK) return chk;
    return gdn::launch_chunk_backward(b, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK
                                                                                       : GDN_ERR_HIP;
}

GDN_EXPORT size_t gdn_kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N,
                                                    int varlen, int chunk, int dtype) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return 0;
    if (chunk != 64 || !head_dim_ok(dk) || !head_dim_ok(dv)) return 0;
    if (shape_check(B, T, H, dk, dv, N, varlen != 0) != GDN_OK) return 0;
    return gdn::kda_workspace_layout(B, T, H, dk, N, varlen != 0, dtype == GDN_BF16 ? 2 : 4).total;
}

namespace {
// Shared by the channel-wise-decay entry points: beta, or the erase and write gates.
int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g_log_alpha,
                  const float* beta, const float* erase, const float* write, const float* h0, void* o,
                  float* hT, const int32_t* cu_seqlens, int chunk, int B, int T, int H, int dk, int dv,
                  int N, int dtype, int o_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (o_dtype != GDN_F32 && !(o_dtype == GDN_BF16 && dtype == GDN_BF16)) return GDN_ERR_DTYPE;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    const int sc = shape_check(B, T, H, dk, dv, N, cu_seqlens != nullptr);
    if (sc != GDN_OK) return sc;
    const long long tokens = (long long)B * T;
    if (tokens > 0 && (!q || !k || !v || !g_log_alpha || !o || (!erase && !beta) || (erase && !write)))
        return GDN_ERR_NULL;
    const void* al16[] = {q, k, v, o, h0, hT, g_log_alpha, erase, write};
    for (const void* x : al16)
        if (x && !aligned(x, 16)) return GDN_ERR_ALIGN;
    const void* al4[] = {beta, cu_seqlens};
    for (const void* x : al4)
        if (x && !aligned(x, 4)) return GDN_ERR_ALIGN;
    const gdn::KdaLayout w = gdn::kda_workspace_layout(B, T, H, dk, N, cu_seqlens != nullptr, dtype == GDN_BF16 ? 2 : 4);
    if (w.nc_bound * H > 0x7fffffffL) return GDN_ERR_SHAPE;
    if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return GDN_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 256)) return GDN_ERR_ALIGN;
    char* base = static_cast<char*>(workspace);
    gdn::ChunkProblem P{};
    P.q = q; P.k = k; P.v = v; P.g = g_log_alpha; P.beta = beta; P.h0 = h0; P.o = o; P.hT = hT;
    P.cu_seqlens = cu_seqlens;
    P.B = B; P.T = T; P.H = H; P.dk = dk; P.dv = dv; P.N = N;
    P.bf16 = dtype == GDN_BF16;
    P.o_bf16 = o_dtype == GDN_BF16;
    P.nc_bound = w.nc_bound;
    P.nc_per_seq = (T + 63) / 64;
    const bool any = w.nc_bound > 0;
    P.chunk_base = cu_seqlens ? reinterpret_cast<int32_t*>(base + w.off_base) : nullptr;
    P.mmat = any ? base + w.off_m : nullptr;
    P.pmat = any ? base + w.off_p : nullptr;
    P.khat = any ? reinterpret_cast<float*>(base + w.off_kh) : nullptr;
    P.qhat = any ? reinterpret_cast<float*>(base + w.off_qh) : nullptr;
    P.kdec = any ? reinterpret_cast<float*>(base + w.off_kd) : nullptr;
    P.lam = any ? reinterpret_cast<float*>(base + w.off_lam) : nullptr;
    P.erase = erase;
    P.write = erase ? write : nullptr;
    const int chk = debug_check_offsets(cu_seqlens, N, T, static_cast<hipStream_t>(stream));
    if (chk != GDN_OK) return chk;
    return gdn::launch_kda_chunk_fwd(P, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK
                                                                                       : GDN_ERR_HIP;
}
}  // namespace

GDN_EXPORT int gdn_kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g_log_alpha,
                                 const float* beta, const float* h0, void* o, float* hT,
                                 const int32_t* cu_seqlens, int chunk, int B, int T, int H, int dk,
                                 int dv, int N, int dtype, int o_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return kda_chunk_fwd(q, k, v, g_log_alpha, beta, nullptr, nullptr, h0, o, hT, cu_seqlens, chunk, B, T,
                         H, dk, dv, N, dtype, o_dtype, workspace, workspace_bytes, stream);
}

GDN_EXPORT int gdn_decoupled_chunk_fwd(const void* q, const void* k, const void* v, const float* g_log_alpha,
                                       const float* erase, const float* write, const float* h0, void* o,
                                       float* hT, const int32_t* cu_seqlens, int chunk, int B, int T, int H,
                                       int dk, int dv, int N, int dtype, int o_dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (B * (long long)T > 0 && (!erase || !write)) return GDN_ERR_NULL;
    return kda_chunk_fwd(q, k, v, g_log_alpha, nullptr, erase, write, h0, o, hT, cu_seqlens, chunk, B, T,
                         H, dk, dv, N, dtype, o_dtype, workspace, workspace_bytes, stream);
}

GDN_EXPORT int gdn_kda_decode_step(const void* q, const void* k, const void* v, const float* g_log_alpha,
                                   const float* beta, float* state, void* o, int N, int H, int dk,
                                   int dv, int dtype, int o_dtype, void* stream) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (o_dtype != GDN_F32 && o_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    if (N < 1 || H < 1 || (long long)N * H > 0x7fffffffLL) return GDN_ERR_SHAPE;
    if (!q || !k || !v || !g_log_alpha || !beta || !state || !o) return GDN_ERR_NULL;
    const void* al16[] = {q, k, v, o, state, g_log_alpha};
    for (const void* x : al16)
        if (!aligned(x, 16)) return GDN_ERR_ALIGN;
    if (!aligned(beta, 4)) return GDN_ERR_ALIGN;
    gdn::DecodeProblem p{q,  k, v,  g_log_alpha, beta,           state,
                         o,  N, H,  dk,          dv,   dtype == GDN_BF16, o_dtype == GDN_BF16};
    p.channel_gate = 1;
    return gdn::launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK
                                                                                : GDN_ERR_HIP;
}

GDN_EXPORT int gdn_decoupled_decode_step(const void* q, const void* k, const void* v, const float* g_log_alpha,
                                         const float* erase, const float* write, float* state, void* o, int N,
                                         int H, int dk, int dv, int dtype, int o_dtype, void* stream) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (o_dtype != GDN_F32 && o_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    if (N < 1 || H < 1 || (long long)N * H > 0x7fffffffLL) return GDN_ERR_SHAPE;
    if (!q || !k || !v || !g_log_alpha || !erase || !write || !state || !o) return GDN_ERR_NULL;
    const void* al16[] = {q, k, v, o, state, g_log_alpha, erase, write};
    for (const void* x : al16)
        if (!aligned(x, 16)) return GDN_ERR_ALIGN;
    gdn::DecodeProblem p{q,  k, v,  g_log_alpha, nullptr,        state,
                         o,  N, H,  dk,          dv,   dtype == GDN_BF16, o_dtype == GDN_BF16};
    p.channel_gate = 1;
    p.erase = erase;
    p.write = write;
    return gdn::launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK
                                                                                : GDN_ERR_HIP;
}
