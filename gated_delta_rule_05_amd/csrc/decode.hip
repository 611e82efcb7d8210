// decode.hip -- one KDA decode step on gfx950: each head state streams
// through HBM exactly once.
//
// Per (sequence, head), with S the fp32 d_k x d_v state (d_v contiguous):
//     S~ = Diag(alpha) S,  r_k = S~^T k,  r_q = S~^T q,
//     e  = beta (v - r_k),
//     o  = scale (r_q + e (k . q)),          (= scale * (S~ + k e^T)^T q)
//     S  <- S~ + k e^T                        (in place)
// which is one token of the recurrence in "Kimi Delta Attention: la
// atencion lineal detras de Kimi K2 y Qwen3", section "Cómo funciona Kimi
// Delta Attention paso a paso".  Reading the output from the two
// reductions of the decayed state, instead of re-reading the corrected
// state, is what lets the kernel touch S once: one 128-bit load and one
// 128-bit store per 4 state elements.
//
// Mapping: one work-group per head state.  Each wave owns CW = min(d_v, 32)
// whole columns of the state; a lane holds 4 adjacent columns of every
// (64 / (CW/4))-th row, so a wave instruction covers full 128-byte rows
// segments, and both reductions over d_k finish inside the wave with
// cross-lane shuffles (no LDS, no barrier).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename T, int DK, int DV>
__global__ __launch_bounds__((DV < 32 ? 1 : DV / 32) * 64)
void decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                        const T* __restrict__ v, const float* __restrict__ log_alpha,
                        const float* __restrict__ beta, float* __restrict__ S,
                        T* __restrict__ o, float scale)
{
    constexpr int CW = DV < 32 ? DV : 32;   // state columns per wave
    constexpr int LPR = CW / 4;             // lanes sharing one row
    constexpr int RPI = 64 / LPR;           // rows covered per wave instruction
    constexpr int ITERS = DK / RPI;         // rows per lane
    static_assert(DK % RPI == 0, "d_k must be a multiple of the rows per instruction");

    const int64_t nh = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int col = wave * CW + (lane % LPR) * 4;
    const int row0 = lane / LPR;

    float* Sp = S + nh * (DK * DV);
    const T* qp = q + nh * DK;
    const T* kp = k + nh * DK;
    const float* lap = log_alpha + nh * DK;

    f32x4 s[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) s[it] = load_stream4(Sp + (row0 + it * RPI) * DV + col);

    float rk0 = 0.f, rk1 = 0.f, rk2 = 0.f, rk3 = 0.f;
    float rq0 = 0.f, rq1 = 0.f, rq2 = 0.f, rq3 = 0.f;
    float kq = 0.f;
    float kr[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int r = row0 + it * RPI;
        const float a = gate_exp(lap[r]);
        const float kv = elem<T>::load(kp + r);
        const float qv = elem<T>::load(qp + r);
        kr[it] = kv;
        kq += kv * qv;
        s[it].x *= a; s[it].y *= a; s[it].z *= a; s[it].w *= a;
        rk0 += kv * s[it].x; rk1 += kv * s[it].y; rk2 += kv * s[it].z; rk3 += kv * s[it].w;
        rq0 += qv * s[it].x; rq1 += qv * s[it].y; rq2 += qv * s[it].z; rq3 += qv * s[it].w;
    }
    // sum over the lanes that hold the other rows of the same columns
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
        rk0 += __shfl_xor(rk0, m); rk1 += __shfl_xor(rk1, m);
        rk2 += __shfl_xor(rk2, m); rk3 += __shfl_xor(rk3, m);
        rq0 += __shfl_xor(rq0, m); rq1 += __shfl_xor(rq1, m);
        rq2 += __shfl_xor(rq2, m); rq3 += __shfl_xor(rq3, m);
        kq += __shfl_xor(kq, m);
    }
    const float b = beta[nh];
    const float4 vv = elem<T>::load4(v + nh * DV + col);
    const float e0 = b * (vv.x - rk0), e1 = b * (vv.y - rk1);
    const float e2 = b * (vv.z - rk2), e3 = b * (vv.w - rk3);
    if (row0 == 0) {
        elem<T>::store4(o + nh * DV + col,
                        make_float4(scale * (rq0 + e0 * kq), scale * (rq1 + e1 * kq),
                                    scale * (rq2 + e2 * kq), scale * (rq3 + e3 * kq)));
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        f32x4 x = s[it];
        x.x += kr[it] * e0; x.y += kr[it] * e1; x.z += kr[it] * e2; x.w += kr[it] * e3;
        store_stream4(Sp + (row0 + it * RPI) * DV + col, x);
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int threads = (DV < 32 ? 1 : DV / 32) * 64;
    const int64_t blocks = static_cast<int64_t>(a.N) * a.H;
    hipLaunchKernelGGL((decode_step_kernel<T, DK, DV>), dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), 0, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.log_alpha, a.beta, a.S,
                       static_cast<T*>(a.o), a.scale);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_decode_dv(const DecodeArgs& a, hipStream_t stream) {
    switch (a.d_v) {
        case 16: return launch_decode_t<T, DK, 16>(a, stream);
        case 32: return launch_decode_t<T, DK, 32>(a, stream);
        case 64: return launch_decode_t<T, DK, 64>(a, stream);
        case 128: return launch_decode_t<T, DK, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_dk(const DecodeArgs& a, hipStream_t stream) {
    switch (a.d_k) {
        case 16: return launch_decode_dv<T, 16>(a, stream);
        case 32: return launch_decode_dv<T, 32>(a, stream);
        case 64: return launch_decode_dv<T, 64>(a, stream);
        case 128: return launch_decode_dv<T, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.dtype_f32) return launch_decode_dk<float>(a, stream);
    return launch_decode_dk<bf16_t>(a, stream);
}

}  // namespace kda
