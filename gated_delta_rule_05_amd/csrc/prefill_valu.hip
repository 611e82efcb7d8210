// prefill_valu.hip -- chunked KDA prefill with fp32 vector arithmetic.
//
// This is the exact-precision path: fp32 inputs (and any shape the matrix
// core path does not cover) run here, with every product, the triangular
// solve and the state in fp32.  It computes the same chunked (UT / WY) form
// as the matrix-core kernel, so it also checks that algebra at a tight
// tolerance.
//
// Chunked form (the pages only say the recurrence is evaluated blockwise
// with a diagonal-plus-low-rank transition -- "Kimi Linear acaba de superar
// a la atención completa en sus propios términos", section "Cómo Kimi
// Linear utiliza una memoria recurrente más inteligente"; the algebra below
// is derived from the per-token recurrence).  For a chunk of C tokens with
// start state S0 (d_k x d_v), per key channel c:
//   g_r   = sum_{s<=r} log_alpha_s            (cumulative gate inside the chunk)
//   Kg    = K * e^{g},  Qg = Q * e^{g},  Kn = K * e^{-g},  Kd = K * e^{g_C - g}
//   A     = strictly-lower(Diag(beta) Kg Kn^T)     the chunk's delta-rule system
//   P     = lower(Qg Kn^T)                         (diagonal included)
//   E     = (I + A)^{-1} Diag(beta) (V - Kg S0)    the delta errors of the chunk
//   O     = scale (Qg S0 + P E)
//   S_C   = Diag(e^{g_C}) S0 + Kd^T E
// The rows of S never mix in any of these maps, so each work-group owns a
// tile of TV state columns (value channels) and the tiles run in parallel.
//
// Any gate: where a chunk's cumulative gate leaves the factored form's range,
// A and P are summed entry by entry with their own factors e^{g_r - g_s}
// from fp64 cumulative gates (see the kernel).
//
// One work-group of 256 threads per (sequence, head, value tile) walks the
// sequence's chunks in order; the last chunk is masked (rows past the end
// carry k = q = v = 0, log_alpha = 0, beta = 0, so they change nothing).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_sched.h"

namespace kda {

// |g| (natural log units) up to which the factored form e^{g} e^{-g} runs:
// its factors then stay far inside fp32, and their relative error (about
// |g| 2^-23 each) inside the fp32 parity bar
constexpr float kSafeGate = 16.f;

template <typename T, int DK, int TV, int C>
__global__ __launch_bounds__(256)
void prefill_valu_kernel(const T* __restrict__ q, const T* __restrict__ k,
                         const T* __restrict__ v, const float* __restrict__ log_alpha,
                         const float* __restrict__ beta, const float* __restrict__ h0,
                         const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
                         int64_t groups, int R, int H, int DV, float scale,
                         T* __restrict__ o, float* __restrict__ hT, int gate,
                         float* __restrict__ snapshots, int snap_tokens, int snap_cap,
                         FrontEnd fe)
{
    constexpr int NT = 256;
    constexpr int KP = DK + 1;   // padded row stride: column walks hit distinct banks
    __shared__ float sKg[C * KP], sQg[C * KP], sKn[C * KP], sKd[C * KP];
    __shared__ float sA[C * C], sP[C * C], sTi[C * C];
    __shared__ float sS[DK * TV], sV[C * TV], sX[C * TV], sE[C * TV];
    __shared__ float sBeta[C], sGl[DK], sGe[DK];
    __shared__ float sNk[C], sNq[C];   // front-end: 1 / ||k||, 1 / ||q|| per row
    // the exact form (below): cumulative gates in fp64, so that differences
    // g_r - g_s keep full fp32 precision however long the decay
    __shared__ double sGd[C * KP], sGdl[DK];
    __shared__ int sExact;

    int64_t pair;
    int tile;
    if (!prefill_map_block(blockIdx.x, groups, R, pair, tile)) return;
    const int tid = threadIdx.x;
    const int h = static_cast<int>(pair % H);
    const int n = order[pair / H];
    const int64_t t_begin = cu[n];
    const int64_t t_end = cu[n + 1];
    const int j0 = tile * TV;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV + j0;

    for (int i = tid; i < DK * TV; i += NT) {
        const int c = i / TV, j = i % TV;
        sS[i] = h0 ? h0[sbase + static_cast<int64_t>(c) * DV + j] : 0.f;
    }

    int snap_left = snapshots ? snap_tokens / C : 0;
    for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
        const int len = static_cast<int>(min<int64_t>(C, t_end - c0));
        __syncthreads();
        // stage k, q and log_alpha (masked past the end of the sequence)
        for (int i = tid; i < C * DK; i += NT) {
            const int r = i / DK, c = i % DK;
            float kk = 0.f, qq = 0.f, la = 0.f;
            if (r < len) {
                const int64_t off = ((c0 + r) * H + h) * DK + c;
                kk = elem<T>::load(k + off);
                qq = elem<T>::load(q + off);
                // the key channel's own gate, the head's (broadcast) or none;
                // with the front-end, from its bf16 pre-activation
                if (fe.gate_pre) {
                    const int64_t go = gate == kGateChannel ? off : (c0 + r) * H + h;
                    la = gate == kGateNone ? 0.f
                                           : -fe.gate_scale * softplus_f32(bf16_to_f32(fe.gate_pre[go]));
                } else {
                    la = gate == kGateChannel ? log_alpha[off]
                         : gate == kGateHead  ? log_alpha[(c0 + r) * H + h]
                                              : 0.f;
                }
            }
            sKg[r * KP + c] = kk;
            sQg[r * KP + c] = qq;
            sKn[r * KP + c] = la;
        }
        for (int i = tid; i < C * TV; i += NT) {
            const int r = i / TV, j = i % TV;
            sV[i] = (r < len) ? elem<T>::load(v + ((c0 + r) * H + h) * DV + j0 + j) : 0.f;
        }
        for (int r = tid; r < C; r += NT)
            sBeta[r] = r >= len ? 0.f
                       : fe.beta_pre ? sigmoid_f32(bf16_to_f32(fe.beta_pre[(c0 + r) * H + h]))
                                     : beta[(c0 + r) * H + h];
        __syncthreads();
        if (fe.l2norm) {
            // front-end: each row of k and q divided by its L2 norm
            for (int r = tid; r < C; r += NT) {
                float sk = 0.f, sq = 0.f;
                for (int c = 0; c < DK; ++c) {
                    sk += sKg[r * KP + c] * sKg[r * KP + c];
                    sq += sQg[r * KP + c] * sQg[r * KP + c];
                }
                sNk[r] = 1.f / fmaxf(sqrtf(sk), kFrontEps);
                sNq[r] = 1.f / fmaxf(sqrtf(sq), kFrontEps);
            }
            __syncthreads();
            for (int i = tid; i < C * DK; i += NT) {
                const int r = i / DK, c = i % DK;
                sKg[r * KP + c] *= sNk[r];
                sQg[r * KP + c] *= sNq[r];
            }
            __syncthreads();
        }
        // cumulative gate per key channel; a chunk where some |g| leaves the
        // range of the factored form (or is NaN) takes the exact form
        if (tid == 0) sExact = 0;
        __syncthreads();
        for (int c = tid; c < DK; c += NT) {
            float g = 0.f;
            double gd = 0.0;
            bool wild = false;
            for (int r = 0; r < C; ++r) {
                const float la = sKn[r * KP + c];
                g += la;
                gd += static_cast<double>(la);
                sKn[r * KP + c] = g;
                sGd[r * KP + c] = gd;
                wild |= !(fabsf(g) <= kSafeGate);
            }
            sGl[c] = g;
            sGdl[c] = gd;
            sGe[c] = gate_exp(g);
            if (wild) sExact = 1;
        }
        __syncthreads();
        const bool exact = sExact != 0;
        if (exact) {
            // A and P entry by entry: every factor e^{g_r - g_s} (s <= r) is
            // at most 1 and is formed from an fp64 difference, so no decay is
            // out of range and none loses precision
            for (int i = tid; i < C * C; i += NT) {
                const int r = i / C, s = i % C;
                float a = 0.f, p = 0.f;
                if (s <= r) {
                    for (int c = 0; c < DK; ++c) {
                        const float e = gate_exp(static_cast<float>(sGd[r * KP + c] - sGd[s * KP + c]));
                        const float w = sKg[s * KP + c] * e;
                        a += sKg[r * KP + c] * w;
                        p += sQg[r * KP + c] * w;
                    }
                    a = (s < r) ? sBeta[r] * a : 0.f;
                }
                sA[i] = a;
                sP[i] = p;
            }
            __syncthreads();
        }
        // decay-weighted copies of k and q
        for (int i = tid; i < C * DK; i += NT) {
            const int r = i / DK, c = i % DK;
            const float g = sKn[r * KP + c];
            const float kk = sKg[r * KP + c];
            const float eg = gate_exp(g);
            const float emg = gate_exp(-g);
            sKg[r * KP + c] = kk * eg;
            sQg[r * KP + c] = sQg[r * KP + c] * eg;
            sKn[r * KP + c] = kk * emg;
            sKd[r * KP + c] = kk * (exact ? gate_exp(static_cast<float>(sGdl[c] - sGd[r * KP + c]))
                                          : gate_exp(sGl[c] - g));
        }
        __syncthreads();
        // A (strictly lower, rows scaled by beta) and P (lower, with diagonal)
        for (int i = tid; i < C * C && !exact; i += NT) {
            const int r = i / C, s = i % C;
            float a = 0.f, p = 0.f;
            if (s <= r) {
                const float* kg = sKg + r * KP;
                const float* qg = sQg + r * KP;
                const float* kn = sKn + s * KP;
                for (int c = 0; c < DK; ++c) {
                    a += kg[c] * kn[c];
                    p += qg[c] * kn[c];
                }
                a = (s < r) ? sBeta[r] * a : 0.f;
            }
            sA[i] = a;
            sP[i] = p;
        }
        __syncthreads();
        // Ti = (I + A)^{-1} by forward substitution, one column per thread
        for (int col = tid; col < C; col += NT) {
            for (int r = 0; r < C; ++r) {
                float x = (r == col) ? 1.f : 0.f;
                if (r > col) {
                    for (int s = col; s < r; ++s) x -= sA[r * C + s] * sTi[s * C + col];
                }
                sTi[r * C + col] = x;
            }
        }
        __syncthreads();
        // X = Diag(beta) (V - Kg S0)
        for (int i = tid; i < C * TV; i += NT) {
            const int r = i / TV, j = i % TV;
            float acc = 0.f;
            for (int c = 0; c < DK; ++c) acc += sKg[r * KP + c] * sS[c * TV + j];
            sX[i] = sBeta[r] * (sV[i] - acc);
        }
        __syncthreads();
        // E = (I + A)^{-1} X
        for (int i = tid; i < C * TV; i += NT) {
            const int r = i / TV, j = i % TV;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc += sTi[r * C + s] * sX[s * TV + j];
            sE[i] = acc;
        }
        __syncthreads();
        // O = scale (Qg S0 + P E)
        for (int i = tid; i < C * TV; i += NT) {
            const int r = i / TV, j = i % TV;
            if (r < len) {
                float acc = 0.f;
                for (int c = 0; c < DK; ++c) acc += sQg[r * KP + c] * sS[c * TV + j];
                for (int s = 0; s <= r; ++s) acc += sP[r * C + s] * sE[s * TV + j];
                elem<T>::store(o + ((c0 + r) * H + h) * DV + j0 + j, scale * acc);
            }
        }
        __syncthreads();
        // S_C = Diag(e^{g_C}) S0 + Kd^T E
        for (int i = tid; i < DK * TV; i += NT) {
            const int c = i / TV, j = i % TV;
            float acc = sGe[c] * sS[i];
            for (int r = 0; r < C; ++r) acc += sKd[r * KP + c] * sE[r * TV + j];
            sS[i] = acc;
        }
        // a snapshot after every snap_tokens / C chunks (each thread copies
        // the state entries it has just written)
        const int js = snapshots && --snap_left == 0
                           ? (snap_left = snap_tokens / C, static_cast<int>((c0 + len - t_begin) / snap_tokens) - 1)
                           : -1;
        if (js >= 0 && js < snap_cap && len == C) {      // only a full chunk ends on a boundary
            float* dst = snapshot_at(snapshots, snap_cap, H, static_cast<int64_t>(DK) * DV, n, js, h) + j0;
            for (int i = tid; i < DK * TV; i += NT) dst[(i / TV) * DV + i % TV] = sS[i];
        }
    }
    if (hT) {
        __syncthreads();
        for (int i = tid; i < DK * TV; i += NT) {
            const int c = i / TV, j = i % TV;
            hT[sbase + static_cast<int64_t>(c) * DV + j] = sS[i];
        }
    }
}

template <typename T, int DK, int TV>
static hipError_t launch_valu_t(const PrefillArgs& a, int R, hipStream_t stream) {
    constexpr int C = 32;
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    const int64_t blocks = prefill_grid_blocks(groups, R);
    hipLaunchKernelGGL((prefill_valu_kernel<T, DK, TV, C>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.log_alpha, a.beta, a.h0,
                       a.cu_seqlens, a.order, groups, R, a.H, a.d_v, a.scale,
                       static_cast<T*>(a.o), a.hT, a.gate, a.snapshots, a.snap_tokens, a.snap_cap,
                       a.fe);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_valu_dk(const PrefillArgs& a, hipStream_t stream) {
    if (a.d_v == 16) return launch_valu_t<T, DK, 16>(a, 1, stream);
    return launch_valu_t<T, DK, 32>(a, a.d_v / 32, stream);
}

template <typename T>
static hipError_t launch_valu(const PrefillArgs& a, hipStream_t stream) {
    switch (a.d_k) {
        case 16: return launch_valu_dk<T, 16>(a, stream);
        case 32: return launch_valu_dk<T, 32>(a, stream);
        case 64: return launch_valu_dk<T, 64>(a, stream);
        case 128: return launch_valu_dk<T, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_valu(const PrefillArgs& a, hipStream_t stream) {
    if (a.dtype_f32) return launch_valu<float>(a, stream);
    return launch_valu<bf16_t>(a, stream);
}

}  // namespace kda
