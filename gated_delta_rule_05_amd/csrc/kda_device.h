// kda_device.h -- small device helpers shared by the gfx950 KDA kernels:
// element conversions (bf16 <-> fp32, round to nearest even), vector loads
// and stores of 4 elements, and the exponential used for the gates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef uint16_t bf16_t;  // raw bf16 bits as stored in memory
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte state accesses that bypass cache retention: each state element
// is read once and written once per call, so keeping it in L2 only evicts
// data that is reused.
__device__ __forceinline__ f32x4 load_stream4(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store_stream4(float* p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Element access for the two supported input types.
template <typename T> struct elem;
template <> struct elem<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
    // 4 consecutive elements (16-byte aligned)
    __device__ __forceinline__ static float4 load4(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
    __device__ __forceinline__ static void store4(float* p, float4 x) {
        *reinterpret_cast<float4*>(p) = x;
    }
};
template <> struct elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
    // 4 consecutive elements (8-byte aligned)
    __device__ __forceinline__ static float4 load4(const bf16_t* p) {
        uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
    __device__ __forceinline__ static void store4(bf16_t* p, float4 x) {
        uint2 u;
        u.x = pack_bf16x2(x.x, x.y);
        u.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<uint2*>(p) = u;
    }
};

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^-|x|), through the
// hardware base-2 exponential and logarithm (the second term is in (0, ln 2])
__device__ __forceinline__ float softplus_f32(float x) {
    const float t = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    return fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + t) * 0.6931471805599453f;
}

// sigmoid(x) = 1 / (1 + e^-x)
__device__ __forceinline__ float sigmoid_f32(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// exp(x) through the hardware base-2 exponential.  Relative error is a few
// ulp plus |x| * 2^-24 from scaling x by log2(e); |x| stays below ~90 on
// every factored path that calls it; in a chunk beyond that range only its
// values for x <= 0 are used (they underflow to 0 as e^x does).
__device__ __forceinline__ float gate_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace kda
