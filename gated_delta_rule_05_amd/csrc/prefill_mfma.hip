// prefill_mfma.hip -- chunked KDA prefill on gfx950 matrix cores (bf16
// operands, fp32 accumulation, fp32 state), d_k = 128, chunks of 64 tokens.
//
// Per chunk of C = 64 tokens with start state S0 (d_k x d_v, fp32), per key
// channel c (derived from the per-token recurrence; the pages only say it is
// evaluated blockwise with a diagonal-plus-low-rank transition):
//   g_r  = sum_{s<=r} log_alpha_s
//   Kg   = K * e^{g},  Qg = Q * e^{g},  Kn = K * e^{-g},  Kd = Kn * e^{g_last}
//   A    = strictly-lower(Diag(beta) Kg Kn^T)        (C x C)
//   P    = lower(Qg Kn^T)                            (C x C, diagonal included)
//   X    = Diag(beta) (V - Kg S0)
//   E    : (I + A) E = X                             the chunk's delta errors
//   O    = scale (Qg S0 + P E)
//   S    = Diag(e^{g_last}) S0 + Kd^T E
//
// Work split.  One work-group (4 waves) per (sequence, head, value tile of
// TV columns).  Per chunk:
//   1. all waves: load k, q, log_alpha, beta and the V tile, cumulative gate,
//      exponentials, write Kg, Qg, Kn, Kd^T (bf16) to LDS;
//   2. all waves: A on MFMA (10 lower 16x16 tiles);
//   3. wave 0: fp32 inverses of the four 16x16 diagonal blocks of I + A
//      (forward substitution, one column per lane); waves 1-3: P on MFMA;
//   4. the serial part, per 16-column slab of the state, entirely in the
//      owning wave's registers: Y = Kg S0, X, block forward substitution for
//      E, O, and the state update.
// The state never leaves registers between chunks.  Its fp32 tiles sit in
// the accumulator layout (lane l holds rows 4(l/16)+i of column l%16); to
// use them as the K operand of the next product, the K index of both
// operands is permuted the same way (K-step kk takes rows 32kk + 4g + i and
// 32kk + 16 + 4g + i from the lane group g = l/16), which leaves each
// product unchanged.  For the 16x16x16 products of the substitution the
// accumulator layout already is the B-operand layout.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_sched.h"

namespace kda {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;        // tokens per chunk
constexpr int DK = 128;      // key channels
constexpr int NT = 256;      // threads per work-group
constexpr int KS = DK + 8;   // bf16 row stride of Kg / Qg / Kn
constexpr int RS = C + 8;    // bf16 row stride of Kd^T, -A, P
constexpr int DS = 20;       // bf16 row stride of the diagonal-block inverses
constexpr int AS = 17;       // fp32 row stride of the diagonal blocks of A

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
__device__ __forceinline__ float unbf(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
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

// A-operand fragment of a bf16 row with the permuted K order of K-step kk
__device__ __forceinline__ u32x4 perm_row(const uint16_t* row, int kk, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 32 * kk + 4 * g);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 32 * kk + 16 + 4 * g);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// the ten lower-triangular 16x16 tiles (I, J), J <= I, of a 64x64 matrix,
// numbered row by row: job = I (I + 1) / 2 + J
__device__ __forceinline__ int tile_row(int job) { return (job >= 1) + (job >= 3) + (job >= 6); }
__device__ __forceinline__ int tile_col(int job) {
    const int I = tile_row(job);
    return job - I * (I + 1) / 2;
}

template <int TV>
struct alignas(16) Smem {
    uint16_t kg[C * KS];
    uint16_t qg[C * KS];
    uint16_t kn[C * KS];
    uint16_t kdt[DK * RS];
    uint16_t an[C * RS];          // -A, bf16; upper blocks stay zero
    uint16_t p[C * RS];           // P, bf16; upper blocks stay zero
    uint16_t dinv[4 * 16 * DS];   // (I + A_II)^{-1}, bf16, [block][row][col]
    float adiag[4 * 16 * AS];     // A_II, fp32, [block][row][col]
    uint16_t v[C * (TV + 8)];
    float beta[C];
    float gam[DK];                // e^{g_last} per key channel
    float tot[4 * DK];            // per-quarter gate sums
};

}  // namespace

template <int TV>
__global__ __launch_bounds__(NT)
void prefill_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                         const bf16_t* __restrict__ v, const float* __restrict__ log_alpha,
                         const float* __restrict__ beta, const float* __restrict__ h0,
                         const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
                         int64_t groups, int R, int H, int DV, float scale,
                         bf16_t* __restrict__ o, float* __restrict__ hT)
{
    constexpr int NSLAB = TV / 16;                  // 16-column slabs in the tile
    constexpr int SPW = NSLAB >= 4 ? NSLAB / 4 : 1; // slabs per active wave
    constexpr int VS = TV + 8;
    __shared__ Smem<TV> sm;

    int64_t pair;
    int tile;
    if (!prefill_map_block(blockIdx.x, groups, R, pair, tile)) return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int h = static_cast<int>(pair % H);
    const int n = order[pair / H];
    const int64_t t_begin = cu[n];
    const int64_t t_end = cu[n + 1];
    const int j0 = tile * TV;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV + j0;
    const bool active = wave < NSLAB;

    for (int i = tid; i < C * RS / 2; i += NT) {
        reinterpret_cast<uint32_t*>(sm.an)[i] = 0u;
        reinterpret_cast<uint32_t*>(sm.p)[i] = 0u;
    }

    // fp32 state of this wave's slabs, accumulator layout:
    // S[sl][m][i] = state[c = 16m + 4g + i][j = (wave + 4 sl) * 16 + ln]
    f32x4 S[SPW][8];
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jc = (wave + 4 * sl) * 16 + ln;
                S[sl][m][i] = (h0 && active)
                    ? h0[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc] : 0.f;
            }

    for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
        const int len = static_cast<int>(min<int64_t>(C, t_end - c0));
        __syncthreads();

        // ---- 1. gates and decay-weighted operands ----------------------
        {
            const int cp = tid & 63;     // key channels 2cp, 2cp+1
            const int qr = tid >> 6;     // rows 16qr .. 16qr+15
            float kx[16], ky[16], qx[16], qy[16], gx[16], gy[16];
            float run0 = 0.f, run1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 16 * qr + r;
                // rows past the end read row 0 of the chunk and are zeroed
                const bool valid = row < len;
                const int64_t off = ((c0 + (valid ? row : 0)) * H + h) * DK + 2 * cp;
                uint32_t kv = *reinterpret_cast<const uint32_t*>(k + off);
                uint32_t qv = *reinterpret_cast<const uint32_t*>(q + off);
                float2 la = *reinterpret_cast<const float2*>(log_alpha + off);
                if (!valid) {
                    kv = 0u;
                    qv = 0u;
                    la = make_float2(0.f, 0.f);
                }
                kx[r] = __uint_as_float(kv << 16);
                ky[r] = __uint_as_float(kv & 0xffff0000u);
                qx[r] = __uint_as_float(qv << 16);
                qy[r] = __uint_as_float(qv & 0xffff0000u);
                run0 += la.x;
                run1 += la.y;
                gx[r] = run0;
                gy[r] = run1;
            }
            sm.tot[qr * DK + 2 * cp] = run0;
            sm.tot[qr * DK + 2 * cp + 1] = run1;
            if (tid < C) sm.beta[tid] = (tid < len) ? beta[(c0 + tid) * H + h] : 0.f;
            for (int i = tid; i < C * TV / 4; i += NT) {
                const int r = i / (TV / 4), j4 = (i % (TV / 4)) * 4;
                uint2 vv = make_uint2(0u, 0u);
                if (r < len)
                    vv = *reinterpret_cast<const uint2*>(v + ((c0 + r) * H + h) * DV + j0 + j4);
                *reinterpret_cast<uint2*>(sm.v + r * VS + j4) = vv;
            }
            __syncthreads();
            float pre0 = 0.f, pre1 = 0.f, last0 = 0.f, last1 = 0.f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float t0 = sm.tot[qq * DK + 2 * cp], t1 = sm.tot[qq * DK + 2 * cp + 1];
                if (qq < qr) { pre0 += t0; pre1 += t1; }
                last0 += t0;
                last1 += t1;
            }
            const float gl0 = gate_exp(last0), gl1 = gate_exp(last1);
            if (qr == 0) {
                sm.gam[2 * cp] = gl0;
                sm.gam[2 * cp + 1] = gl1;
            }
            uint32_t kd0[8], kd1[8];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 16 * qr + r;
                const float g0 = pre0 + gx[r], g1 = pre1 + gy[r];
                const float e0 = gate_exp(g0), e1 = gate_exp(g1);
                const float n0 = gate_exp(-g0), n1 = gate_exp(-g1);
                *reinterpret_cast<uint32_t*>(sm.kg + row * KS + 2 * cp) = pk(kx[r] * e0, ky[r] * e1);
                *reinterpret_cast<uint32_t*>(sm.qg + row * KS + 2 * cp) = pk(qx[r] * e0, qy[r] * e1);
                *reinterpret_cast<uint32_t*>(sm.kn + row * KS + 2 * cp) = pk(kx[r] * n0, ky[r] * n1);
                const float d0 = kx[r] * n0 * gl0, d1 = ky[r] * n1 * gl1;
                if (r & 1) {
                    kd0[r >> 1] |= static_cast<uint32_t>(bf(d0)) << 16;
                    kd1[r >> 1] |= static_cast<uint32_t>(bf(d1)) << 16;
                } else {
                    kd0[r >> 1] = bf(d0);
                    kd1[r >> 1] = bf(d1);
                }
            }
            u32x4* t0 = reinterpret_cast<u32x4*>(sm.kdt + (2 * cp) * RS + 16 * qr);
            u32x4* t1 = reinterpret_cast<u32x4*>(sm.kdt + (2 * cp + 1) * RS + 16 * qr);
            t0[0] = u32x4{kd0[0], kd0[1], kd0[2], kd0[3]};
            t0[1] = u32x4{kd0[4], kd0[5], kd0[6], kd0[7]};
            t1[0] = u32x4{kd1[0], kd1[1], kd1[2], kd1[3]};
            t1[1] = u32x4{kd1[4], kd1[5], kd1[6], kd1[7]};
        }
        __syncthreads();

        // ---- 2. A = strictly-lower(Diag(beta) Kg Kn^T) -----------------
        for (int job = wave; job < 10; job += 4) {
            const int I = tile_row(job), J = tile_col(job);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(sm.kg + (16 * I + ln) * KS + 32 * kk + 8 * g);
                const u32x4 b = *reinterpret_cast<const u32x4*>(sm.kn + (16 * J + ln) * KS + 32 * kk + 8 * g);
                acc = mma32(a, b, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * g + i, s = 16 * J + ln;
                const float br = sm.beta[r];
                const float val = (r > s) ? br * acc[i] : 0.f;
                sm.an[r * RS + s] = bf(-val);
                if (I == J) sm.adiag[(I * 16 + 4 * g + i) * AS + ln] = val;
            }
        }
        __syncthreads();

        // ---- 3. diagonal-block inverses (wave 0) and P (waves 1-3) ------
        if (wave == 0) {
            // lane = 16 * block + column; forward substitution down the rows
            const float* ab = sm.adiag + g * 16 * AS;
            float d[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = (r == ln) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) x -= ab[r * AS + s] * d[s];
                d[r] = x;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.dinv[(g * 16 + r) * DS + ln] = bf(d[r]);
        } else {
            for (int job = wave - 1; job < 10; job += 3) {
                const int I = tile_row(job), J = tile_col(job);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(sm.qg + (16 * I + ln) * KS + 32 * kk + 8 * g);
                    const u32x4 b = *reinterpret_cast<const u32x4*>(sm.kn + (16 * J + ln) * KS + 32 * kk + 8 * g);
                    acc = mma32(a, b, acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * g + i, s = 16 * J + ln;
                    sm.p[r * RS + s] = bf((r >= s) ? acc[i] : 0.f);
                }
            }
        }
        __syncthreads();

        // ---- 4. serial part, one 16-column slab at a time ---------------
        if (active) {
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) {
                const int jc = (wave + 4 * sl) * 16 + ln;   // column within the tile
                u32x4 sb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) sb[kk] = pack4(S[sl][2 * kk], S[sl][2 * kk + 1]);

                // X = Diag(beta) (V - Kg S0)
                f32x4 X[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const uint16_t* row = sm.kg + (16 * I + ln) * KS;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) acc = mma32(perm_row(row, kk, g), sb[kk], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * I + 4 * g + i;
                        X[I][i] = sm.beta[r] * (unbf(sm.v[r * VS + jc]) - acc[i]);
                    }
                }
                // (I + A) E = X by block forward substitution
                u32x2 eb[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    f32x4 z = X[I];
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        const u32x2 a = *reinterpret_cast<const u32x2*>(sm.an + (16 * I + ln) * RS + 16 * J + 4 * g);
                        z = mma16(a, eb[J], z);
                    }
                    const u32x2 d = *reinterpret_cast<const u32x2*>(sm.dinv + (I * 16 + ln) * DS + 4 * g);
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    eb[I] = pack2(mma16(d, pack2(z), zero));
                }
                // O = scale (Qg S0 + P E)
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const uint16_t* qrow = sm.qg + (16 * I + ln) * KS;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) acc = mma32(perm_row(qrow, kk, g), sb[kk], acc);
                    const uint16_t* prow = sm.p + (16 * I + ln) * RS;
#pragma unroll
                    for (int ss = 0; ss < 2; ++ss) {
                        if (ss == 1 && I < 2) continue;
                        const u32x4 b = u32x4{eb[2 * ss][0], eb[2 * ss][1], eb[2 * ss + 1][0], eb[2 * ss + 1][1]};
                        acc = mma32(perm_row(prow, ss, g), b, acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * I + 4 * g + i;
                        if (r < len) o[((c0 + r) * H + h) * DV + j0 + jc] = bf(scale * acc[i]);
                    }
                }
                // S = Diag(e^{g_last}) S0 + Kd^T E
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    f32x4 acc;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = sm.gam[16 * m + 4 * g + i] * S[sl][m][i];
                    const uint16_t* krow = sm.kdt + (16 * m + ln) * RS;
#pragma unroll
                    for (int ss = 0; ss < 2; ++ss) {
                        const u32x4 b = u32x4{eb[2 * ss][0], eb[2 * ss][1], eb[2 * ss + 1][0], eb[2 * ss + 1][1]};
                        acc = mma32(perm_row(krow, ss, g), b, acc);
                    }
                    S[sl][m] = acc;
                }
            }
        }
    }

    if (hT && active) {
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int jc = (wave + 4 * sl) * 16 + ln;
                    hT[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc] = S[sl][m][i];
                }
    }
}

template <int TV>
static hipError_t launch_mfma_t(const PrefillArgs& a, int R, hipStream_t stream) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    const int64_t blocks = prefill_grid_blocks(groups, R);
    hipLaunchKernelGGL((prefill_mfma_kernel<TV>), dim3(static_cast<unsigned>(blocks)), dim3(NT),
                       0, stream, static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.log_alpha, a.beta, a.h0, a.cu_seqlens,
                       a.order, groups, R, a.H, a.d_v, a.scale, static_cast<bf16_t*>(a.o), a.hT);
    return hipGetLastError();
}

bool mfma_supported(const PrefillArgs& a) { return !a.dtype_f32 && a.d_k == DK; }

// Value tiles per (sequence, head): enough work-groups to cover the 256
// compute units, but tiles no narrower than 16 columns.
int mfma_value_tiles(const PrefillArgs& a) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    int R = 1;
    while (R < a.d_v / 16 && groups * R < 256) R *= 2;
    return R;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int R, hipStream_t stream) {
    switch (a.d_v / R) {
        case 16: return launch_mfma_t<16>(a, R, stream);
        case 32: return launch_mfma_t<32>(a, R, stream);
        case 64: return launch_mfma_t<64>(a, R, stream);
        case 128: return launch_mfma_t<128>(a, R, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
