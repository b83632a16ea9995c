// Device helpers for the gfx950 (CDNA4) kernels: bf16 conversion, MFMA tile products
// and small vector loads. Included only by the .hip sources of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kWave = 64;    // CDNA wavefront width

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename TS> __device__ __forceinline__ TS from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

// ------------------------------------------------------------- MFMA fragments
// A fragment holds, for one lane, 8 consecutive values along the contraction index k.
// In a 16x16 output tile, lane l supplies row (l % 16) of the left operand and column
// (l % 16) of the right operand, for k = 8 * (l / 16) + 0..7 of each 32-wide k slice.
// Any relabelling of k is harmless as long as both operands use the same one, which
// every caller below does by loading both from the same k offsets.
template <typename TS> struct Frag;
template <> struct Frag<uint16_t> { uint4 v; };            // 8 x bf16
template <> struct Frag<float> { float4 lo, hi; };          // 8 x fp32

template <typename TS>
__device__ __forceinline__ Frag<TS> load_frag(const TS* p);
template <>
__device__ __forceinline__ Frag<uint16_t> load_frag<uint16_t>(const uint16_t* p) {
    Frag<uint16_t> f;
    f.v = *reinterpret_cast<const uint4*>(p);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag<float>(const float* p) {
    Frag<float> f;
    f.lo = *reinterpret_cast<const float4*>(p);
    f.hi = *reinterpret_cast<const float4*>(p + 4);
    return f;
}

// d (16x16 fp32 accumulator tile, 4 values per lane: rows 4*(l/16)+0..3, column l%16)
// += A[16 x 32] * B[32 x 16] for one 32-wide k slice.
__device__ __forceinline__ void mma_k32(f32x4_t& d, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), d, 0, 0, 0);
}
// fp32 operands: eight 16x16x4 products. Step s uses, in lane l, k = 8*(l/16) + s, which
// covers the same 32 k values as the bf16 form.
__device__ __forceinline__ void mma_k32(f32x4_t& d, const Frag<float>& a, const Frag<float>& b) {
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, d, 0, 0, 0);
}

// d += A * Bt^T over a K-long contraction ("NT" product). a_row points at this lane's
// row of A (row l%16 of the tile), b_row at this lane's row of Bt (column l%16 of the
// tile); both are contiguous along k.
template <typename TS, int K>
__device__ __forceinline__ void mma_nt(f32x4_t& d, const TS* a_row, const TS* b_row) {
    const int kq = 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32)
        mma_k32(d, load_frag<TS>(a_row + k0 + kq), load_frag<TS>(b_row + k0 + kq));
}

// Gather 8 values at a fixed column from 8 consecutive rows (stride in elements).
template <typename TS>
__device__ __forceinline__ Frag<TS> gather_frag(const TS* p, int stride);
template <>
__device__ __forceinline__ Frag<uint16_t> gather_frag<uint16_t>(const uint16_t* p, int stride) {
    Frag<uint16_t> f;
    f.v.x = (uint32_t)p[0] | ((uint32_t)p[stride] << 16);
    f.v.y = (uint32_t)p[2 * stride] | ((uint32_t)p[3 * stride] << 16);
    f.v.z = (uint32_t)p[4 * stride] | ((uint32_t)p[5 * stride] << 16);
    f.v.w = (uint32_t)p[6 * stride] | ((uint32_t)p[7 * stride] << 16);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> gather_frag<float>(const float* p, int stride) {
    Frag<float> f;
    f.lo = make_float4(p[0], p[stride], p[2 * stride], p[3 * stride]);
    f.hi = make_float4(p[4 * stride], p[5 * stride], p[6 * stride], p[7 * stride]);
    return f;
}

// Store 4 consecutive values (one accumulator column run) as TS.
template <typename TS>
__device__ __forceinline__ void store4(TS* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    u.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
    *reinterpret_cast<uint2*>(p) = u;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Store 16 consecutive values (given as fp32) as TS with 16-byte vector stores.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}
template <typename TS>
__device__ __forceinline__ void store16(TS* dst, const float (&x)[16]);
template <>
__device__ __forceinline__ void store16<uint16_t>(uint16_t* dst, const float (&x)[16]) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pack_bf16x2(x[8], x[9]), pack_bf16x2(x[10], x[11]),
                                                    pack_bf16x2(x[12], x[13]), pack_bf16x2(x[14], x[15]));
}
template <>
__device__ __forceinline__ void store16<float>(float* dst, const float (&x)[16]) {
#pragma unroll
    for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
}

// 16 bytes of zeros / a 16-byte vector copy, used for tiles staged through registers.
__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace gdn
