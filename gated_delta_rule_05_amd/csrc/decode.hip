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
// Mapping: a persistent grid of work-groups, each walking head states
// g, g + G, g + 2G, ...; NWV waves per work-group, each owning whole rows
// (key channels) of the state: a lane holds 4 adjacent columns of every
// (256 / d_v)-th row of its wave's rows, so each wave instruction reads or
// writes whole 512-byte rows (contiguous 1 KB at d_v = 128) with
// non-temporal 128-bit accesses.  While a work-group reduces and writes
// back one head, the loads of its next head are already in flight, so the
// state streams without a gap between reading and writing.  The column
// reductions over d_k finish with cross-lane shuffles inside each wave and
// one exchange of the per-wave partial sums through LDS (double-buffered,
// so one barrier per head).
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int LPR = DV / 4;                       // lanes sharing one row
    static constexpr int RPI = 64 / LPR;                     // rows per wave instruction
    static constexpr int PER = 16;                           // rows per lane (at most)
    static constexpr int NWV = DK / RPI > PER ? DK / RPI / PER : 1;   // waves
    static constexpr int ITERS = DK / (NWV * RPI);           // rows per lane
    static_assert(ITERS >= 1 && ITERS * NWV * RPI == DK, "rows split evenly");
};

constexpr int kDecodeGrid = 256;   // persistent work-groups (one per compute unit)

// FRONT: the fused input front-end (its own instantiation): gates from
// bf16 pre-activations (log_alpha = -fe.gate_scale softplus(x)), beta =
// sigmoid of a bf16 pre-activation, and q, k divided by their L2 norms,
// which are reduced together with k . q and applied after the reductions
// (the reductions are linear in q and k)
template <typename T, int DK, int DV, int GATE, bool INDEXED, bool FRONT>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NWV * 64))
void decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                        const T* __restrict__ v, const float* __restrict__ log_alpha,
                        const float* __restrict__ beta, float* __restrict__ S,
                        T* __restrict__ o, float scale, int64_t nheads, int H,
                        const int32_t* __restrict__ state_index, int num_states, FrontEnd fe)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int LPR = Sh::LPR, RPI = Sh::RPI, NWV = Sh::NWV, ITERS = Sh::ITERS;
    __shared__ f32x4 red[2][NWV][2][LPR];   // per-wave column partials of S~^T k and S~^T q
    __shared__ float red_kq[2][NWV];
    __shared__ float red_nrm[FRONT ? 2 : 1][NWV][2];   // front-end: sum of k^2 and q^2

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int cl = lane % LPR;                // 4 columns: 4cl .. 4cl+3
    const int row0 = wave * (ITERS * RPI) + lane / LPR;
    // head nh = (sequence n, head h) keeps its state in slot state_index[n]
    // (or n); a slot outside [0, num_states) marks a skipped sequence, whose
    // loads read slot 0 and whose results are dropped
    auto slot = [&](int64_t nh) -> int64_t {
        if constexpr (!INDEXED) {
            // the 256 work-groups work on consecutive heads together; visit
            // the sequences in the order n -> (n * 97) mod N (a bijection
            // when N is not a multiple of 97) so that the states streamed
            // at the same time lie far apart in memory (1.3 % faster than
            // one contiguous window, measured)
            const int64_t n = nh / H, nseq = nheads / H;
            const int64_t ns = nseq % 97 ? (n * 97) % nseq : n;
            return ns * H + (nh - n * H);
        }
        const int64_t n = nh / H;
        const int32_t x = state_index[n];
        return x >= 0 && x < num_states ? static_cast<int64_t>(x) * H + (nh - n * H) : -1;
    };
    auto state = [&](int64_t sh, int it) {
        return S + (sh < 0 ? 0 : sh) * (DK * DV) + (row0 + it * RPI) * DV + 4 * cl;
    };

    int64_t nh = blockIdx.x;
    if (nh >= nheads) return;
    f32x4 s[ITERS], sn[ITERS];
    int64_t sh = slot(nh);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) s[it] = load_stream4(state(sh, it));
    for (int par = 0; nh < nheads; nh += gridDim.x, par ^= 1) {
        // next head's state (this head again past the end: same data, never stored)
        const int64_t nn = nh + gridDim.x < nheads ? nh + gridDim.x : nh;
        const int64_t shn = slot(nn);
#pragma unroll
        for (int it = 0; it < ITERS; ++it) sn[it] = load_stream4(state(shn, it));

        const int64_t nx = INDEXED ? nh : sh;      // the token inputs of the scrambled sequence
        const T* qp = q + nx * DK;
        const T* kp = k + nx * DK;
        // the gate of key channel r: its own (KDA), the head's (Gated
        // DeltaNet) or none (DeltaNet: alpha = 1)
        const bool pre = FRONT && fe.gate_pre;
        const float la_head = GATE != kGateHead ? 0.f
                              : pre ? -fe.gate_scale * softplus_f32(bf16_to_f32(fe.gate_pre[nx]))
                              : log_alpha ? log_alpha[nx] : 0.f;
        auto la_of = [&](int r) {
            if constexpr (GATE == kGateChannel) {
                if (pre) return -fe.gate_scale * softplus_f32(bf16_to_f32(fe.gate_pre[nx * DK + r]));
                return log_alpha[nx * DK + r];
            } else {
                return la_head;
            }
        };
        f32x4 rk = {0.f, 0.f, 0.f, 0.f}, rq = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f, kk = 0.f, qq = 0.f;
        float kr[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int r = row0 + it * RPI;
            const float a = gate_exp(la_of(r));
            const float kv = elem<T>::load(kp + r);
            const float qv = elem<T>::load(qp + r);
            kr[it] = kv;
            kq += kv * qv;
            if constexpr (FRONT) {
                kk += kv * kv;
                qq += qv * qv;
            }
            s[it] *= a;
            rk += kv * s[it];
            rq += qv * s[it];
        }
        // sum over the lanes of this wave that hold other rows of the same columns
#pragma unroll
        for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rk[c] += __shfl_xor(rk[c], m);
                rq[c] += __shfl_xor(rq[c], m);
            }
            kq += __shfl_xor(kq, m);
            if constexpr (FRONT) {
                kk += __shfl_xor(kk, m);
                qq += __shfl_xor(qq, m);
            }
        }
        if (NWV > 1) {
            // ... and over the waves
            if (lane < LPR) {
                red[par][wave][0][cl] = rk;
                red[par][wave][1][cl] = rq;
                if (lane == 0) red_kq[par][wave] = kq;
                if (FRONT && lane == 0) {
                    red_nrm[FRONT ? par : 0][wave][0] = kk;
                    red_nrm[FRONT ? par : 0][wave][1] = qq;
                }
            }
            __syncthreads();
            rk = red[par][0][0][cl];
            rq = red[par][0][1][cl];
            kq = red_kq[par][0];
            if constexpr (FRONT) {
                kk = red_nrm[par][0][0];
                qq = red_nrm[par][0][1];
            }
#pragma unroll
            for (int w = 1; w < NWV; ++w) {
                rk += red[par][w][0][cl];
                rq += red[par][w][1][cl];
                kq += red_kq[par][w];
                if constexpr (FRONT) {
                    kk += red_nrm[par][w][0];
                    qq += red_nrm[par][w][1];
                }
            }
        }
        if constexpr (FRONT) {
            // the reductions are linear in k and q: normalise them afterwards
            if (fe.l2norm) {
                const float ik = 1.f / fmaxf(sqrtf(kk), kFrontEps);
                const float iq = 1.f / fmaxf(sqrtf(qq), kFrontEps);
                rk *= ik;
                rq *= iq;
                kq *= ik * iq;
#pragma unroll
                for (int it = 0; it < ITERS; ++it) kr[it] *= ik;
            }
        }
        const float b = FRONT && fe.beta_pre ? sigmoid_f32(bf16_to_f32(fe.beta_pre[nx])) : beta[nx];
        const float4 vv = elem<T>::load4(v + nx * DV + 4 * cl);
        const f32x4 e = {b * (vv.x - rk[0]), b * (vv.y - rk[1]), b * (vv.z - rk[2]),
                         b * (vv.w - rk[3])};
        if (!INDEXED || sh >= 0) {
            if (wave == 0 && lane < LPR) {
                const f32x4 oo = scale * (rq + kq * e);
                elem<T>::store4(o + nx * DV + 4 * cl, make_float4(oo[0], oo[1], oo[2], oo[3]));
            }
#pragma unroll
            for (int it = 0; it < ITERS; ++it) store_stream4(state(sh, it), s[it] + kr[it] * e);
        }
#pragma unroll
        for (int it = 0; it < ITERS; ++it) s[it] = sn[it];
        sh = shn;
    }
}

// Several tokens per sequence (m, stored [N][m][H][.]), applied in order to
// the state held in registers: one read of each state for all of them.
// Sequence n applies its first len_n = clamp(lengths[n], 0, m) tokens (all
// m without lengths), writes the outputs of those tokens when o is given,
// and stores the state after them when write_state is set.  Speculative
// decoding uses it twice: to verify m draft tokens (outputs only, the state
// left as it was) and to commit the accepted prefix (state only).  Each
// token is the same arithmetic as decode_step_kernel's single token, in the
// same order, so a commit of m tokens equals m decode steps bit for bit.
// one lane's share of a token's inputs: its rows of k, q and the gate, its
// 4 columns of v, and beta
template <int ITERS>
struct DecodeTok {
    float kv[ITERS], qv[ITERS], la[ITERS];
    float b;
    float4 vv;
};

// FRONT: the fused input front-end, per token as in decode_step_kernel
// (activations at load; norms reduced with k . q and applied after the
// reductions), so m tokens still equal m single steps bit for bit
template <typename T, int DK, int DV, int GATE, bool INDEXED, bool FRONT>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NWV * 64))
void decode_multi_kernel(const T* __restrict__ q, const T* __restrict__ k,
                         const T* __restrict__ v, const float* __restrict__ log_alpha,
                         const float* __restrict__ beta, float* __restrict__ S,
                         T* __restrict__ o, float scale, int64_t nheads, int H, int m,
                         const int32_t* __restrict__ lengths, int write_state,
                         const int32_t* __restrict__ state_index, int num_states, FrontEnd fe)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int LPR = Sh::LPR, RPI = Sh::RPI, NWV = Sh::NWV, ITERS = Sh::ITERS;
    using Tok = DecodeTok<ITERS>;
    __shared__ f32x4 red[2][NWV][2][LPR];
    __shared__ float red_kq[2][NWV];
    __shared__ float red_nrm[FRONT ? 2 : 1][NWV][2];   // front-end: sum of k^2 and q^2

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int cl = lane % LPR;
    const int row0 = wave * (ITERS * RPI) + lane / LPR;
    auto slot = [&](int64_t nh) -> int64_t {
        if constexpr (!INDEXED) return nh;
        const int64_t n = nh / H;
        const int32_t x = state_index[n];
        return x >= 0 && x < num_states ? static_cast<int64_t>(x) * H + (nh - n * H) : -1;
    };
    auto state = [&](int64_t sh, int it) {
        return S + (sh < 0 ? 0 : sh) * (DK * DV) + (row0 + it * RPI) * DV + 4 * cl;
    };

    // No prefetch of the next head's state (unlike the single step): the
    // registers go to the next token's inputs instead, and two work-groups
    // per compute unit overlap one's loads with the other's token steps.
    int par = 0;
    for (int64_t nh = blockIdx.x; nh < nheads; nh += gridDim.x) {
        const int64_t sh = slot(nh);
        f32x4 s[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) s[it] = load_stream4(state(sh, it));

        const int64_t n = nh / H;
        const int64_t h = nh - n * H;
        const int len = lengths ? min(max(lengths[n], 0), m) : m;
        const bool live = !INDEXED || sh >= 0;
        // the inputs of token i+1 load while token i computes, so a head
        // pays the memory latency of its token inputs about once, not m
        // times
        auto load_tok = [&](Tok& t, int i) {
            const int64_t tk = (n * m + i) * H + h;      // token row
            const T* qp = q + tk * DK;
            const T* kp = k + tk * DK;
            const bool pre = FRONT && fe.gate_pre;
            const float la_head = GATE != kGateHead ? 0.f
                                  : pre ? -fe.gate_scale * softplus_f32(bf16_to_f32(fe.gate_pre[tk]))
                                  : log_alpha ? log_alpha[tk] : 0.f;
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const int r = row0 + it * RPI;
                if constexpr (GATE == kGateChannel) {
                    t.la[it] = pre ? -fe.gate_scale * softplus_f32(bf16_to_f32(fe.gate_pre[tk * DK + r]))
                                   : log_alpha[tk * DK + r];
                } else {
                    t.la[it] = la_head;
                }
                t.kv[it] = elem<T>::load(kp + r);
                t.qv[it] = elem<T>::load(qp + r);
            }
            t.b = FRONT && fe.beta_pre ? sigmoid_f32(bf16_to_f32(fe.beta_pre[tk])) : beta[tk];
            t.vv = elem<T>::load4(v + tk * DV + 4 * cl);
        };
        Tok cur, nxt;
        if (len > 0) load_tok(cur, 0);
        for (int i = 0; i < len; ++i) {
            if (i + 1 < len) load_tok(nxt, i + 1);
            const int64_t tk = (n * m + i) * H + h;
            f32x4 rk = {0.f, 0.f, 0.f, 0.f}, rq = {0.f, 0.f, 0.f, 0.f};
            float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const float a = gate_exp(cur.la[it]);
                kq += cur.kv[it] * cur.qv[it];
                if constexpr (FRONT) {
                    kk += cur.kv[it] * cur.kv[it];
                    qq += cur.qv[it] * cur.qv[it];
                }
                s[it] *= a;
                rk += cur.kv[it] * s[it];
                rq += cur.qv[it] * s[it];
            }
#pragma unroll
            for (int mk = LPR; mk < 64; mk <<= 1) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    rk[c] += __shfl_xor(rk[c], mk);
                    rq[c] += __shfl_xor(rq[c], mk);
                }
                kq += __shfl_xor(kq, mk);
                if constexpr (FRONT) {
                    kk += __shfl_xor(kk, mk);
                    qq += __shfl_xor(qq, mk);
                }
            }
            if (NWV > 1) {
                // double-buffered by a parity that flips per reduction: the
                // barrier of the next one keeps a fast wave from overwriting
                // partials a slow wave is still reading
                if (lane < LPR) {
                    red[par][wave][0][cl] = rk;
                    red[par][wave][1][cl] = rq;
                    if (lane == 0) red_kq[par][wave] = kq;
                    if (FRONT && lane == 0) {
                        red_nrm[FRONT ? par : 0][wave][0] = kk;
                        red_nrm[FRONT ? par : 0][wave][1] = qq;
                    }
                }
                __syncthreads();
                rk = red[par][0][0][cl];
                rq = red[par][0][1][cl];
                kq = red_kq[par][0];
                if constexpr (FRONT) {
                    kk = red_nrm[par][0][0];
                    qq = red_nrm[par][0][1];
                }
#pragma unroll
                for (int w = 1; w < NWV; ++w) {
                    rk += red[par][w][0][cl];
                    rq += red[par][w][1][cl];
                    kq += red_kq[par][w];
                    if constexpr (FRONT) {
                        kk += red_nrm[par][w][0];
                        qq += red_nrm[par][w][1];
                    }
                }
                par ^= 1;
            }
            float ik = 1.f;                              // the key's normalisation
            if constexpr (FRONT) {
                if (fe.l2norm) {
                    ik = 1.f / fmaxf(sqrtf(kk), kFrontEps);
                    const float iq = 1.f / fmaxf(sqrtf(qq), kFrontEps);
                    rk *= ik;
                    rq *= iq;
                    kq *= ik * iq;
                }
            }
            const float b = cur.b;
            const float4 vv = cur.vv;
            const f32x4 e = {b * (vv.x - rk[0]), b * (vv.y - rk[1]), b * (vv.z - rk[2]),
                             b * (vv.w - rk[3])};
            if (o && live && wave == 0 && lane < LPR) {
                const f32x4 oo = scale * (rq + kq * e);
                elem<T>::store4(o + tk * DV + 4 * cl, make_float4(oo[0], oo[1], oo[2], oo[3]));
            }
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                float kn = cur.kv[it];
                if constexpr (FRONT) kn *= ik;
                s[it] = s[it] + kn * e;
            }
            cur = nxt;
        }
        if (write_state && live && len > 0) {
#pragma unroll
            for (int it = 0; it < ITERS; ++it) store_stream4(state(sh, it), s[it]);
        }
    }
}

template <typename T, int DK, int DV, int GATE, bool INDEXED, bool FRONT>
static hipError_t launch_step_f(const DecodeArgs& a, int64_t grid, int threads, hipStream_t stream) {
    const int64_t nheads = static_cast<int64_t>(a.N) * a.H;
    hipLaunchKernelGGL((decode_step_kernel<T, DK, DV, GATE, INDEXED, FRONT>),
                       dim3(static_cast<unsigned>(grid)), dim3(threads), 0, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.log_alpha, a.beta, a.S,
                       static_cast<T*>(a.o), a.scale, nheads, a.H, a.state_index,
                       a.num_states, a.fe);
    return hipGetLastError();
}

template <typename T, int DK, int DV, int GATE, bool INDEXED>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t stream) {
    constexpr int threads = DecodeShape<DK, DV>::NWV * 64;
    const int64_t nheads = static_cast<int64_t>(a.N) * a.H;
    // persistent grid; small states (one wave each) get more work-groups
    const int64_t grid = std::min<int64_t>(nheads, kDecodeGrid * (threads == 64 ? 4 : 1));
    if (a.m > 0) {
        // two work-groups per compute unit: one's serial token steps hide
        // the other's latencies (measured: m = 4 verify 271 -> 184 us at
        // 256 sequences x 32 heads, d = 128)
        const int64_t mgrid = std::min<int64_t>(nheads, 2 * grid);
        auto kern = a.fe.active() ? decode_multi_kernel<T, DK, DV, GATE, INDEXED, true>
                                  : decode_multi_kernel<T, DK, DV, GATE, INDEXED, false>;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(mgrid)), dim3(threads), 0, stream,
                           static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), a.log_alpha, a.beta, a.S,
                           static_cast<T*>(a.o), a.scale, nheads, a.H, a.m, a.lengths,
                           a.write_state ? 1 : 0, a.state_index, a.num_states, a.fe);
        return hipGetLastError();
    }
    return a.fe.active() ? launch_step_f<T, DK, DV, GATE, INDEXED, true>(a, grid, threads, stream)
                         : launch_step_f<T, DK, DV, GATE, INDEXED, false>(a, grid, threads, stream);
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    // a per-head gate and no gate share one instantiation (no gate: a null
    // log_alpha, read as zero)
    const bool ch = a.gate == kGateChannel;
    if (a.state_index)
        return ch ? launch_decode_g<T, DK, DV, kGateChannel, true>(a, stream)
                  : launch_decode_g<T, DK, DV, kGateHead, true>(a, stream);
    return ch ? launch_decode_g<T, DK, DV, kGateChannel, false>(a, stream)
              : launch_decode_g<T, DK, DV, kGateHead, false>(a, stream);
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
