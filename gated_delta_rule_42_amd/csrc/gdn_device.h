// Device helpers for the gfx950 (CDNA4) kernels: number formats, MFMA tile products and
// small vector moves. Included only by the .hip sources of this library.
//
// Three element types appear in the kernels:
//   input   TIn: float or bf16 (stored as uint16_t)     - q, k, v as the caller gives them
//   operand TM : float or _Float16                     - what the MFMA units multiply
//   output  TO : float or bf16                          - o as the caller asks for it
// bf16 inputs are multiplied as fp16: every bf16 value of magnitude 2^-14 .. 65504 is exactly
// representable in fp16, and the fp32 intermediates that become operands (state, residuals,
// chunk operators) keep 11 significant bits instead of 8. Accumulation is always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;   // tokens per chunk

// operand type used for a given input type
template <typename TIn> struct Operand;
template <> struct Operand<float> { using type = float; };
template <> struct Operand<uint16_t> { using type = _Float16; };

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(uint16_t bf16_bits) { return __uint_as_float((uint32_t)bf16_bits << 16); }

// fp32 -> bf16, round to nearest even (the conversion instruction of gfx950; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values converted and packed by one instruction: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// 16 bytes of input elements -> 16 bytes of operand elements (same element count).
template <typename TIn>
__device__ __forceinline__ uint4 to_operand16(uint4 raw);
template <>
__device__ __forceinline__ uint4 to_operand16<float>(uint4 raw) { return raw; }
template <>
__device__ __forceinline__ uint4 to_operand16<uint16_t>(uint4 raw) {
    auto cv = [](uint32_t w) {   // two bf16 (low, high) -> two fp16
        return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    };
    return make_uint4(cv(raw.x), cv(raw.y), cv(raw.z), cv(raw.w));
}

// ------------------------------------------------------------- MFMA fragments
// A fragment holds, for one lane, 8 consecutive values along the contraction index k.
// In a 16x16 output tile, lane l supplies row (l % 16) of the left operand and column
// (l % 16) of the right operand, for k = 8 * (l / 16) + 0..7 of each 32-wide k slice; the
// accumulator holds rows 4 * (l / 16) + 0..3 of column l % 16. Any relabelling of k is
// harmless as long as both operands use the same one, which every caller ensures by
// loading both from the same k offsets.
template <typename TM> struct Frag;
template <> struct Frag<_Float16> { uint4 v; };            // 8 x fp16
template <> struct Frag<float> { float4 lo, hi; };          // 8 x fp32

template <typename TM>
__device__ __forceinline__ Frag<TM> load_frag(const TM* p);
template <>
__device__ __forceinline__ Frag<_Float16> load_frag<_Float16>(const _Float16* p) {
    Frag<_Float16> f;
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

// d (16x16 fp32 accumulator tile) += A[16 x 32] * B[32 x 16] for one 32-wide k slice.
__device__ __forceinline__ void mma_k32(f32x4_t& d, const Frag<_Float16>& a, const Frag<_Float16>& b) {
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a.v),
                                                __builtin_bit_cast(f16x8_t, b.v), d, 0, 0, 0);
}
// fp32 operands: eight 16x16x4 products. Step s uses, in lane l, k = 8*(l/16) + s, which
// covers the same 32 k values as the 16-bit form.
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
template <typename TM, int K>
__device__ __forceinline__ void mma_nt(f32x4_t& d, const TM* a_row, const TM* b_row) {
    const int kq = 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32)
        mma_k32(d, load_frag<TM>(a_row + k0 + kq), load_frag<TM>(b_row + k0 + kq));
}

// Gather 8 values at a fixed column from 8 consecutive rows (stride in elements).
template <typename TM>
__device__ __forceinline__ Frag<TM> gather_frag(const TM* p, int stride);
template <>
__device__ __forceinline__ Frag<_Float16> gather_frag<_Float16>(const _Float16* p, int stride) {
    const uint16_t* u = reinterpret_cast<const uint16_t*>(p);
    Frag<_Float16> f;
    f.v.x = (uint32_t)u[0] | ((uint32_t)u[stride] << 16);
    f.v.y = (uint32_t)u[2 * stride] | ((uint32_t)u[3 * stride] << 16);
    f.v.z = (uint32_t)u[4 * stride] | ((uint32_t)u[5 * stride] << 16);
    f.v.w = (uint32_t)u[6 * stride] | ((uint32_t)u[7 * stride] << 16);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> gather_frag<float>(const float* p, int stride) {
    Frag<float> f;
    f.lo = make_float4(p[0], p[stride], p[2 * stride], p[3 * stride]);
    f.hi = make_float4(p[4 * stride], p[5 * stride], p[6 * stride], p[7 * stride]);
    return f;
}

// Store 4 consecutive values (one accumulator column run) as TM.
template <typename TM>
__device__ __forceinline__ void store4(TM* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Store 16 consecutive values (given as fp32) as T with 16-byte vector stores.
template <typename T>
__device__ __forceinline__ void store16(T* dst, const float (&x)[16]);
template <>
__device__ __forceinline__ void store16<_Float16>(_Float16* dst, const float (&x)[16]) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]),
                                                pack_f16x2(x[4], x[5]), pack_f16x2(x[6], x[7]));
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pack_f16x2(x[8], x[9]), pack_f16x2(x[10], x[11]),
                                                    pack_f16x2(x[12], x[13]), pack_f16x2(x[14], x[15]));
}
template <>
__device__ __forceinline__ void store16<float>(float* dst, const float (&x)[16]) {
#pragma unroll
    for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
}

__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace gdn
