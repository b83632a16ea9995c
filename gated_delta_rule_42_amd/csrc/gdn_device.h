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

// x, with the compiler made to assume it may have changed: lane-dependent values derived from it
// inside a loop are recomputed where used instead of being hoisted out of the loop and kept
// (or spilled) for its whole length.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

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

// Buffer resources: a wave-uniform base address and a size in bytes. Vector loads through a
// resource take a 32-bit per-lane byte offset; any access at or past the size reads zeros
// and any store there is dropped, which is how the kernels handle a chunk's ragged tail.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;  // raw (unformatted) buffer, 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}
// Four consecutive fp32 values stored as T (bf16: 8 bytes, fp32: 16 bytes).
template <typename T>
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, int off, const f32x4_t& x);
template <>
__device__ __forceinline__ void buf_store4<uint16_t>(__amdgpu_buffer_rsrc_t r, int off, const f32x4_t& x) {
    const u32x2_t v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
template <>
__device__ __forceinline__ void buf_store4<float>(__amdgpu_buffer_rsrc_t r, int off, const f32x4_t& x) {
    const u32x4_t v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// ------------------------------------------------ raw-input products and re-layouts
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// d += A * Bt^T over a K-long contraction for raw bf16 inputs (rows contiguous along k), on
// the bf16 matrix core: the products of bf16 inputs are exact.
template <int K>
__device__ __forceinline__ void mma_nt_in_bf16(f32x4_t& d, const uint16_t* a_row, const uint16_t* b_row) {
    const int kq = 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const uint4 a = *reinterpret_cast<const uint4*>(a_row + k0 + kq);
        const uint4 b = *reinterpret_cast<const uint4*>(b_row + k0 + kq);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                     __builtin_bit_cast(bf16x8_t, b), d, 0, 0, 0);
    }
}

// The same for raw inputs of either type: bf16 on the bf16 matrix core, fp32 on the fp32 one.
template <typename TIn, int K>
__device__ __forceinline__ void mma_nt_in(f32x4_t& d, const TIn* a_row, const TIn* b_row) {
    if constexpr (sizeof(TIn) == 2) mma_nt_in_bf16<K>(d, a_row, b_row);
    else mma_nt<float, K>(d, a_row, b_row);
}

// A fragment whose 8 k-slots are two runs of 4 consecutive elements: slots 0-3 at p0 and
// slots 4-7 at p1. Used with B fragments packed from two accumulator tiles (pack_frag),
// whose lane holds rows 4*(l/16)+0..3 of each tile.
template <typename TM>
__device__ __forceinline__ Frag<TM> load_frag2(const TM* p0, const TM* p1);
template <>
__device__ __forceinline__ Frag<_Float16> load_frag2<_Float16>(const _Float16* p0, const _Float16* p1) {
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    Frag<_Float16> f;
    f.v = make_uint4(a.x, a.y, b.x, b.y);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag2<float>(const float* p0, const float* p1) {
    Frag<float> f;
    f.lo = *reinterpret_cast<const float4*>(p0);
    f.hi = *reinterpret_cast<const float4*>(p1);
    return f;
}

// Operand fragment from two accumulator tiles: slots 0-3 = tile a, slots 4-7 = tile b.
template <typename TM>
__device__ __forceinline__ Frag<TM> pack_frag(const f32x4_t& a, const f32x4_t& b);
template <>
__device__ __forceinline__ Frag<_Float16> pack_frag<_Float16>(const f32x4_t& a, const f32x4_t& b) {
    Frag<_Float16> f;
    f.v = make_uint4(pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]), pack_f16x2(b[0], b[1]),
                     pack_f16x2(b[2], b[3]));
    return f;
}
template <>
__device__ __forceinline__ Frag<float> pack_frag<float>(const f32x4_t& a, const f32x4_t& b) {
    Frag<float> f;
    f.lo = make_float4(a[0], a[1], a[2], a[3]);
    f.hi = make_float4(b[0], b[1], b[2], b[3]);
    return f;
}

// Transposed read of a 4-row x 16-column block of a row-major 16-bit array in LDS: lane
// l16 of each 16-lane group receives column l16 of rows 0..3. `blk` is the block's top-left
// element, `pitch` the row pitch in elements. On gfx950 one ds_read_b64_tr_b16 does this:
// lane s of the group reads 4 consecutive columns 4*(s%4).. of row s/4, and the hardware
// hands lane i the four elements of column i.
__device__ __forceinline__ uint2 lds_read_t16(const void* blk, int pitch_elems) {
    const int l16 = threadIdx.x & 15;
    const uint16_t* p = static_cast<const uint16_t*>(blk) + (l16 >> 2) * pitch_elems + 4 * (l16 & 3);
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    return __builtin_bit_cast(uint2, v);
}

// Operand fragment read transposed from a row-major array: slots 0-3 are column l16 of the
// 4 rows at blk0, slots 4-7 of the 4 rows at blk1.
template <typename TM>
__device__ __forceinline__ Frag<TM> load_frag_t(const TM* blk0, const TM* blk1, int pitch);
template <>
__device__ __forceinline__ Frag<_Float16> load_frag_t<_Float16>(const _Float16* blk0, const _Float16* blk1,
                                                                int pitch) {
    const uint2 a = lds_read_t16(blk0, pitch);
    const uint2 b = lds_read_t16(blk1, pitch);
    Frag<_Float16> f;
    f.v = make_uint4(a.x, a.y, b.x, b.y);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag_t<float>(const float* blk0, const float* blk1, int pitch) {
    const int l16 = threadIdx.x & 15;
    Frag<float> f;
    f.lo = make_float4(blk0[l16], blk0[pitch + l16], blk0[2 * pitch + l16], blk0[3 * pitch + l16]);
    f.hi = make_float4(blk1[l16], blk1[pitch + l16], blk1[2 * pitch + l16], blk1[3 * pitch + l16]);
    return f;
}

// Column l16 of a 4-row block of raw inputs, as fp32 (the transposed read above for bf16).
template <typename TIn>
__device__ __forceinline__ float4 load4_t(const TIn* blk, int pitch);
template <>
__device__ __forceinline__ float4 load4_t<uint16_t>(const uint16_t* blk, int pitch) {
    const uint2 u = lds_read_t16(blk, pitch);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
template <>
__device__ __forceinline__ float4 load4_t<float>(const float* blk, int pitch) {
    const int l16 = threadIdx.x & 15;
    return make_float4(blk[l16], blk[pitch + l16], blk[2 * pitch + l16], blk[3 * pitch + l16]);
}

// ---------------------------------------------------------------- 16-bit fragments
// A fragment of 8 16-bit values (bf16 or fp16 bits) as the 16x16x32 MFMA operands take it.
__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two 4-element runs of 16-bit values (8 bytes each) as one fragment.
__device__ __forceinline__ uint4 lds_frag2(const void* p0, const void* p1) {
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    return make_uint4(a.x, a.y, b.x, b.y);
}

// Two transposing reads (see lds_read_t16) as one fragment; each lane passes the address of
// its own 4-element run.
__device__ __forceinline__ uint4 lds_frag2_t(const void* p0, const void* p1) {
    const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
    const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1);
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// fp16 fragment from two accumulator tiles (slots 0-3 = tile a, 4-7 = tile b).
__device__ __forceinline__ uint4 pack_f16_frag(const f32x4_t& a, const f32x4_t& b) {
    return make_uint4(pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]), pack_f16x2(b[0], b[1]),
                      pack_f16x2(b[2], b[3]));
}

// The same as a pair of bf16 fragments hi + lo: hi is x rounded to bf16 and lo is the
// rounding remainder x - hi (exact in fp32) rounded to bf16, so hi + lo carries x to about 16
// significant bits. A product with a bf16 operand taken as hi and lo separately is as accurate
// as one with a 16-bit-mantissa operand.
__device__ __forceinline__ float bf16_lo_half(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_half(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void split_bf16_frag(const f32x4_t& a, const f32x4_t& b, uint4& hi, uint4& lo) {
    hi = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                    pack_bf16x2(b[2], b[3]));
    lo = make_uint4(pack_bf16x2(a[0] - bf16_lo_half(hi.x), a[1] - bf16_hi_half(hi.x)),
                    pack_bf16x2(a[2] - bf16_lo_half(hi.y), a[3] - bf16_hi_half(hi.y)),
                    pack_bf16x2(b[0] - bf16_lo_half(hi.z), b[1] - bf16_hi_half(hi.z)),
                    pack_bf16x2(b[2] - bf16_lo_half(hi.w), b[3] - bf16_hi_half(hi.w)));
}

// Global -> LDS copy of 16 bytes per lane through a buffer resource: lane l writes LDS bytes
// [16 l, 16 l + 16) after the wave-uniform address lds_block, reading global byte offset off
// of the resource (zeros where that is out of range).
// LDS address of a generic pointer to a __shared__ object: the low 32 bits of its flat
// address (taken as an integer, which needs no null check).
typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ lds_void_ptr to_lds(const void* p) {
    return (lds_void_ptr)(uintptr_t)(uint32_t)reinterpret_cast<uintptr_t>(p);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds_block, int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(lds_block), 16, off, 0, 0, 0);
}
// The same from a plain global address: wave-uniform base plus a 32-bit per-lane offset.
__device__ __forceinline__ void dma16g(const char* base, unsigned off, const void* lds_block) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + off), to_lds(lds_block), 16, 0, 0);
}

// ------------------------------------------------------------------ wave scan
// Inclusive prefix sum over the 64 lanes of a wave: shifts within each 16-lane row, then the
// row totals broadcast forward (DPP row_shr and row_bcast).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add_src(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x = dpp_add_src<0x111, 0xF>(x);  // row_shr:1
    x = dpp_add_src<0x112, 0xF>(x);  // row_shr:2
    x = dpp_add_src<0x114, 0xF>(x);  // row_shr:4
    x = dpp_add_src<0x118, 0xF>(x);  // row_shr:8
    x = dpp_add_src<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x = dpp_add_src<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// acc (16x16 fp32 tile) += A[16 x 4] B[4 x 16] on the fp32 matrix core: lane l gives
// A[l % 16][l / 16] and B[l / 16][l % 16]; acc holds rows 4 (l / 16) + 0..3 of column l % 16.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

}  // namespace gdn
