// kda_mfma.h -- helpers shared by the gfx950 matrix-core prefill kernels:
// bf16 packing, the two MFMA shapes they use, and raw buffer resources.
//
// Operand layouts (16x16 output tiles, 64 lanes, lane l = 16 g + ln):
//   mfma_f32_16x16x32_bf16   A: lane holds A[ln][8g .. 8g+7]
//                            B: lane holds B[8g .. 8g+7][ln]
//                            D: lane holds D[4g .. 4g+3][ln]
//   mfma_f32_16x16x16_bf16   A: lane holds A[ln][4g .. 4g+3]
//                            B: lane holds B[4g .. 4g+3][ln]   (= the D layout)
// The kernels feed the 32-deep product with a permuted K order: in K-step
// kk, lane group g supplies K indices 32kk + 4g + {0..3} followed by
// 32kk + 16 + 4g + {0..3}.  Applied to both operands this leaves the
// product unchanged, and it makes two accumulator tiles stacked along K
// (rows 32kk + 4g + i and 32kk + 16 + 4g + i) a ready B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"

namespace kda {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, gfx9 family

// ---- buffer resources: loads and stores with a hardware range check (an
// access past num_records bytes reads zero / is dropped)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kBufferWord3);
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 ld64(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Single-use input streams (the gates a prefill reads once) carry the
// non-temporal cache-policy bit, so they displace less of the workspace data
// that a later pass reads back from the caches.  (Output tiles narrower than
// a cache line keep the default policy: with the bit, partial lines leave
// the cache before the neighbouring tiles fill them, and more bytes are
// written.)
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x2 ld64_stream(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCachePolicyNT));
}
__device__ __forceinline__ u32x4 ld128_stream(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNT));
}
__device__ __forceinline__ uint16_t ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, int off, uint16_t x) {
    __builtin_amdgcn_raw_buffer_store_b16(x, r, off, 0, 0);
}
__device__ __forceinline__ void st64(__amdgpu_buffer_rsrc_t r, int off, u32x2 x) {
    __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, 0);
}
__device__ __forceinline__ void st32(__amdgpu_buffer_rsrc_t r, int off, uint32_t x) {
    __builtin_amdgcn_raw_buffer_store_b32(x, r, off, 0, 0);
}

// round-to-nearest-even pack of two fp32 into a bf16 pair (low half = a)
__device__ __forceinline__ uint32_t pk(float a, float b) {
    bf16x2_t r;
    r[0] = static_cast<__bf16>(a);
    r[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t bf(float a) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}
__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ f32x4 mma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ u32x4 pack4(f32x4 lo, f32x4 hi) {
    return u32x4{pk(lo[0], lo[1]), pk(lo[2], lo[3]), pk(hi[0], hi[1]), pk(hi[2], hi[3])};
}
__device__ __forceinline__ u32x2 pack2(f32x4 x) { return u32x2{pk(x[0], x[1]), pk(x[2], x[3])}; }
__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) { return u32x4{a[0], a[1], b[0], b[1]}; }

// ---- gfx950 LDS transpose read (ds_read_b64_tr_b16).  Each 16-lane group
// exchanges the 8-byte chunks its lanes address: lane 4a + b receives, as
// element e, element b of the chunk addressed by lane 4e + a (a, b, e in
// 0..3; layout measured on the device).  If lane s of a group addresses row
// k0 + s / 4, columns n0 + 4 (s % 4) .. +3 of a row-major bf16 array, lane
// n of the group therefore gets rows k0 .. k0 + 3 of column n0 + n.
__device__ __forceinline__ u32x2 ld_tr4(const uint16_t* p) {
    typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (lds_i16x4)(const_cast<uint16_t*>(p))));
}
// the 16x16x32 operand fragment of lane (g, ln) -- K indices k0 + 8g .. +7
// of column ln -- from a bf16 LDS array stored [k][column] with row stride
// ld (a multiple of 4), x pointing at (k0, column 0): two transpose reads
__device__ __forceinline__ u32x4 frag_tr(const uint16_t* x, int ld, int lane) {
    const int g = lane >> 4, ln = lane & 15;
    const uint16_t* p = x + (8 * g + (ln >> 2)) * ld + 4 * (ln & 3);
    return cat(ld_tr4(p), ld_tr4(p + 4 * ld));
}

}  // namespace kda
