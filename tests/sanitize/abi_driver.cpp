// Host-side checks of libgdn's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// every entry point is called with arguments that its checks reject, including sizes at the
// edges of int and long arithmetic, and must return the documented status without launching
// anything (no device is touched: all pointers are fake, aligned or misaligned on purpose).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "gdn.h"

static int failures = 0;
#define EXPECT(call, want)                                                                        \
    do {                                                                                          \
        const long got_ = (long)(call);                                                           \
        if (got_ != (long)(want)) {                                                               \
            std::fprintf(stderr, "line %d: %s returned %ld, expected %ld\n", __LINE__, #call, got_, \
                         (long)(want));                                                           \
            ++failures;                                                                           \
        }                                                                                         \
    } while (0)

int main() {
    void* P = reinterpret_cast<void*>(uintptr_t(0x100000));   // aligned fake device pointer
    void* M = reinterpret_cast<void*>(uintptr_t(0x100004));   // 4-byte aligned only
    const float* F = static_cast<const float*>(P);
    const int32_t* CU = static_cast<const int32_t*>(P);
    float* Fo = static_cast<float*>(P);

    EXPECT(gdn_version() >= 100, 1);
    for (int s = -10; s <= 1; ++s) EXPECT(gdn_status_string(s) != nullptr, 1);

    // workspace sizes: rejected arguments give 0, extreme shapes neither overflow nor trap
    const int dts[] = {GDN_F32, GDN_BF16};
    for (int dt : dts) {
        EXPECT(gdn_chunk_fwd_workspace_bytes(1, 10, 2, 96, 64, 1, 0, 64, dt), 0);
        EXPECT(gdn_chunk_fwd_workspace_bytes(1, 10, 2, 64, 64, 1, 0, 32, dt), 0);
        EXPECT(gdn_chunk_fwd_workspace_bytes(0, 10, 2, 64, 64, 0, 0, 64, dt), 0);
        EXPECT(gdn_chunk_fwd_workspace_bytes(1, -1, 2, 64, 64, 1, 0, 64, dt), 0);
        EXPECT(gdn_chunk_bwd_workspace_bytes(1, 10, 2, 64, 96, 1, 0, 64, dt), 0);
        EXPECT(gdn_kda_chunk_fwd_workspace_bytes(1, 10, 2, 64, 96, 1, 0, 64, dt), 0);
        const int bigs[][3] = {{INT_MAX, INT_MAX, 32768}, {1, INT_MAX, 32768}, {INT_MAX, 1, 1}, {65536, 65536, 32768}};
        for (auto& b : bigs) {
            EXPECT(gdn_chunk_fwd_workspace_bytes(b[0], b[1], b[2], 128, 128, b[0], 0, 64, dt), 0);
            EXPECT(gdn_chunk_bwd_workspace_bytes(b[0], b[1], b[2], 128, 128, b[0], 0, 64, dt), 0);
            EXPECT(gdn_kda_chunk_fwd_workspace_bytes(b[0], b[1], b[2], 128, 128, b[0], 0, 64, dt), 0);
            EXPECT(gdn_chunk_fwd_workspace_bytes(1, b[1], b[2], 128, 128, INT_MAX, 1, 64, dt), 0);
        }
        EXPECT(gdn_chunk_fwd_workspace_bytes(1, 0, 2, 64, 64, 1, 0, 64, dt), 0);
        EXPECT(gdn_chunk_fwd_workspace_bytes(4, 2048, 16, 128, 128, 4, 0, 64, dt) > 0, 1);
    }

    // chunked forward entry points: each call fails one check
    struct Fwd {
        int (*f)(const void*, const void*, const void*, const float*, const float*, const float*, void*, float*,
                 const int32_t*, int, int, int, int, int, int, int, int, int, void*, size_t, void*);
    };
    const Fwd fwds[] = {{gdn_chunk_fwd}, {gdn_kda_chunk_fwd}};
    for (const Fwd& e : fwds) {
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, 7, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_DTYPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_F32, GDN_BF16, P, 1 << 30, nullptr), GDN_ERR_DTYPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 32, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_UNSUPPORTED);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 80, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_UNSUPPORTED);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 0, 10, 2, 64, 64, 0, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, -5, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 2, 10, 2, 64, 64, 3, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, CU, 64, 2, 10, 2, 64, 64, 2, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, INT_MAX, INT_MAX, 32768, 128, 128, INT_MAX, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, INT_MAX, 32768, 128, 128, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, CU, 64, 1, INT_MAX, 32768, 128, 128, INT_MAX, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(nullptr, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_NULL);
        EXPECT(e.f(P, P, P, F, F, nullptr, nullptr, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_NULL);
        EXPECT(e.f(M, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_ALIGN);
        EXPECT(e.f(P, P, P, F, F, static_cast<const float*>(M), P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_ALIGN);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, nullptr, 0, nullptr), GDN_ERR_WORKSPACE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 16, nullptr), GDN_ERR_WORKSPACE);
    }
    EXPECT(gdn_chunk_fwd_noalloc(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 80, 64, 1, GDN_BF16, GDN_F32, nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_chunk_fwd_noalloc(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, 4096, 32, 128, 128, 1, GDN_F32, GDN_F32, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_fwd_noalloc(P, P, P, F, F, nullptr, P, nullptr, nullptr, 64, 1, INT_MAX, 32768, 128, 128, 1, GDN_BF16, GDN_F32, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_decoupled_chunk_fwd(P, P, P, F, nullptr, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_decoupled_chunk_fwd(P, P, P, F, F, F, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 96, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_UNSUPPORTED);

    // the two stages
    EXPECT(gdn_chunk_prepare(P, P, F, F, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, nullptr, 0, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_prepare(P, nullptr, F, F, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, P, 1 << 30, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_chunk_propagate(P, P, P, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, nullptr, 0, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_propagate(P, P, nullptr, nullptr, P, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_F32, P, 1 << 30, nullptr), GDN_ERR_NULL);

    // backward
    EXPECT(gdn_chunk_bwd(P, P, P, F, F, nullptr, P, nullptr, P, P, P, Fo, Fo, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_BF16, nullptr, 0, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_bwd(P, P, P, F, F, nullptr, nullptr, nullptr, P, P, P, Fo, Fo, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_BF16, GDN_BF16, P, 1 << 30, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_chunk_bwd(P, P, P, F, F, nullptr, P, nullptr, P, P, P, Fo, Fo, nullptr, nullptr, 64, 1, 10, 2, 64, 64, 1, GDN_F32, GDN_BF16, P, 1 << 30, nullptr), GDN_ERR_DTYPE);
    EXPECT(gdn_chunk_bwd(P, P, P, F, F, nullptr, P, nullptr, P, P, P, Fo, Fo, nullptr, nullptr, 64, INT_MAX, INT_MAX, 32768, 128, 128, INT_MAX, GDN_BF16, GDN_BF16, P, 1 << 30, nullptr), GDN_ERR_SHAPE);

    // decode steps
    struct Dec {
        int (*f)(const void*, const void*, const void*, const float*, const float*, float*, void*, int, int, int, int,
                 int, int, void*);
    };
    const Dec decs[] = {{gdn_decode_step}, {gdn_kda_decode_step}};
    for (const Dec& e : decs) {
        EXPECT(e.f(P, P, P, F, F, Fo, P, 0, 2, 64, 64, GDN_BF16, GDN_F32, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, Fo, P, INT_MAX, INT_MAX, 64, 64, GDN_BF16, GDN_F32, nullptr), GDN_ERR_SHAPE);
        EXPECT(e.f(P, P, P, F, F, Fo, P, 2, 2, 64, 32, GDN_BF16, GDN_F32, nullptr), GDN_ERR_UNSUPPORTED);
        EXPECT(e.f(P, P, P, F, F, Fo, P, 2, 2, 64, 64, 9, GDN_F32, nullptr), GDN_ERR_DTYPE);
        EXPECT(e.f(P, P, P, F, F, nullptr, P, 2, 2, 64, 64, GDN_BF16, GDN_F32, nullptr), GDN_ERR_NULL);
        EXPECT(e.f(P, P, M, F, F, Fo, P, 2, 2, 64, 64, GDN_BF16, GDN_F32, nullptr), GDN_ERR_ALIGN);
    }
    EXPECT(gdn_decoupled_decode_step(P, P, P, F, F, nullptr, Fo, P, 2, 2, 64, 64, GDN_BF16, GDN_F32, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_decoupled_decode_step(P, P, P, F, F, F, Fo, P, 0, 2, 64, 64, GDN_BF16, GDN_F32, nullptr), GDN_ERR_SHAPE);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver: all checks passed\n");
    return 0;
}
