// gdn_chunk_fwd_noalloc (declared in include/gdn.h): the chunkwise forward pass for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). It runs gdn_chunk_fwd's kernels with a workspace that is this file's
// device array instead of caller memory, and calls no allocating routine.
#include "gdn.h"
#include "gdn_internal.h"

#include <mutex>

#define GDN_EXPORT extern "C" __attribute__((visibility("default")))

// Each GPU the library runs on holds its own copy of this array until the process ends. In
// host code its name is a stand-in, not a device address: host code only ever uses the
// address hipGetSymbolAddress returns for the current device (kernel arguments, copies).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per device with that
// device current; NULL if the lookup failed or the device index is out of range.
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    return scratch_ptr[dev];
}
}  // namespace

GDN_EXPORT int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g_log_alpha,
                                     const float* beta, const float* h0, void* o, float* hT,
                                     const int32_t* cu_seqlens, int chunk, int B, int T, int H, int dk,
                                     int dv, int N, int dtype, int o_dtype, void* stream) {
    // every argument check runs before any HIP call, as in gdn_chunk_fwd
    const int st = gdn::chunk_fwd_check(q, k, v, g_log_alpha, beta, h0, o, hT, cu_seqlens, chunk, B, T, H, dk,
                                        dv, N, dtype, o_dtype);
    if (st != GDN_OK) return st;
    const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, cu_seqlens != nullptr, chunk, dtype);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0 && (ws = scratch_address()) == nullptr) return GDN_ERR_HIP;
    return gdn::chunk_fwd(q, k, v, g_log_alpha, beta, h0, o, hT, cu_seqlens, chunk, B, T, H, dk, dv, N,
                          dtype, o_dtype, ws, need, stream);
}
