// prefill_mfma.hip -- chunked KDA prefill on gfx950 matrix cores (bf16
// operands, fp32 accumulation, fp32 state), d_k = 128, chunks of 64 tokens.
//
// Per chunk of C = 64 tokens with start state S0 (d_k x d_v, fp32), per key
// channel c (derived from the per-token recurrence; the pages only say it is
// evaluated blockwise with a diagonal-plus-low-rank transition):
//   g_r  = sum_{s<=r} log_alpha_s,  G = g_last (the chunk's total gate)
//   Kg   = K * e^{g},  Qg = Q * e^{g},  Kn = K * e^{-g},  Kd = Kn * e^{G}
//   A    = strictly-lower(Diag(beta) Kg Kn^T)        (C x C)
//   P    = lower(Qg Kn^T)                            (C x C, diagonal included)
//   X    = Diag(beta) (V - Kg S0)
//   E    : (I + A) E = X                             the chunk's delta errors
//   O    = scale (Qg S0 + P E)
//   S    = Diag(e^{G}) S0 + Kd^T E
// The factors e^{g_r - g_s} of the chunked form split at the chunk start, so a
// row's factors depend only on the gates up to that row: an output never
// depends, even in rounding, on tokens after it.
//
// Work split.  One work-group of 8 waves per (sequence, head, value tile of
// TV <= 64 columns).  The tile's 16-column state slabs live in the
// registers of NC "consumer" waves for the whole sequence; the other waves
// are "producers".  Everything that does not depend on the state -- staging
// the chunk, gates, decay-weighted operands, A, P and the inverses of the
// 16x16 diagonal blocks of I + A -- is produced one chunk ahead into a
// double-buffered LDS slot, while the consumers run the state-dependent
// part of the current chunk.  Each chunk takes two lock-step phases:
//   phase 1: consumers  Y = Kg S0, X, E (block forward substitution)
//            stagers    chunk n+1: gates, exponentials, Kg, Qg, Kn, Kd^T
//                       (from registers loaded one chunk earlier), then
//                       issue the global loads of chunk n+2
//   phase 2: consumers  O and the state update
//            producers  chunk n+1: A and P tiles on MFMA; the wave that
//                       computes a diagonal tile of A also inverts I + A_II
//                       on MFMA, from (I + N)^{-1} = (I - N)(I + N^2)
//                       (I + N^4)(I + N^8) for the nilpotent N = A_II;
//                       stagers also sum the gates of their rows of chunk
//                       n+2, which phase 1 of the next chunk needs.
// The four stagers each own 16 consecutive rows of every chunk, one key
// channel pair per lane, so each load instruction reads whole 256-byte rows;
// the gate cumsum runs down the rows in registers, and the offset from the
// rows above comes from the per-block gate sums written one phase earlier.
// All chunk loads and the output stores go through buffer resources whose
// range ends at the chunk's last token, so rows past the end of a sequence
// read zeros and their stores are dropped by the hardware range check.
// The state never leaves registers between chunks.  Its fp32 tiles sit in
// the accumulator layout (lane l holds rows 4(l/16)+i of column l%16); to
// use them as the K operand of the next product, the K index of both
// operands is permuted the same way (K-step kk takes rows 32kk + 4g + i and
// 32kk + 16 + 4g + i from lane group g = l/16), which leaves each product
// unchanged.  For the 16x16x16 products of the substitution the
// accumulator layout already is the B-operand layout.
#include "kda_device.h"
#include "kda_exact.h"
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_sched.h"

namespace kda {
namespace {

constexpr int C = 64;        // tokens per chunk
constexpr int DK = 128;      // key channels
constexpr int NW = 8;        // waves per work-group
constexpr int NT = NW * 64;  // threads per work-group
constexpr int KS = DK + 4;   // bf16 row stride of Kg / Qg / Kn (8-byte aligned rows)
// bf16 row stride of Kd^T and P: 8-byte aligned rows (the operand reads take
// 8-byte pieces), 34 dwords apart, so the stagers' Kd^T stores (one channel
// row per lane, the same token columns) reach 16 bank pairs where a stride of
// C + 8 reached 4, and P's 2-byte stores (rows 4 apart) no bank twice
constexpr int RS = C + 4;
constexpr int DS = 20;       // bf16 row stride of 16x16 blocks (-A off-diagonal, inverses)
constexpr int NSTAGE = 4;    // stager waves, 16 rows of each chunk apiece
constexpr int kMaxTileColumns = 128; // four consumer waves of up to two 16-column slabs
constexpr int kMaxHeads = 16384;     // keeps every chunk-relative byte offset in 31 bits

// A-operand fragment of a bf16 row with the permuted K order of K-step kk
__device__ __forceinline__ u32x4 perm_row(const uint16_t* row, int kk, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 32 * kk + 4 * g);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 32 * kk + 16 + 4 * g);
    return cat(lo, hi);
}

// lower-triangular 16x16 tiles (I, J), J <= I, of a 64x64 matrix, numbered
// row by row: t = I (I + 1) / 2 + J
__device__ __forceinline__ int tile_row(int t) { return (t >= 1) + (t >= 3) + (t >= 6); }
__device__ __forceinline__ int tile_col(int t) {
    const int I = tile_row(t);
    return t - I * (I + 1) / 2;
}
// the six strictly-lower tiles (J < I), numbered I (I - 1) / 2 + J
__device__ __forceinline__ int offdiag_index(int I, int J) { return I * (I - 1) / 2 + J; }

struct alignas(16) Smem {
    uint16_t kg[2][C * KS];            // K * e^{g}
    uint16_t qg[2][C * KS];            // Q * e^{g}
    uint16_t kdt[2][DK * RS];          // (K * e^{G - g})^T
    uint16_t p[2][C * RS];             // P; the upper 16x16 blocks stay zero
    uint16_t an[2][6 * 16 * DS];       // -A, strictly-lower 16x16 blocks
    uint16_t dinv[2][4 * 16 * DS];     // (I + A_II)^{-1}
    float beta[2][C];
    float gam[2][DK];                  // e^{G}
    uint16_t kn[C * KS];               // K * e^{-g} (producers only)
    float2 tot[2][4 * (DK / 2)];       // gate sums of the four 16-row blocks (log2 units)
    int xflag[2];                      // the chunk's form beyond the factored range: 0 none,
                                       // 1 blocked, 2 pairwise
    float nrm[2][2][C];                // front-end: 1 / ||k||, 1 / ||q|| of each row
};

// |g| (log2 units) up to which e^{g} and e^{-g} stay inside fp32 (e^{80}).
// A chunk whose total gate G leaves that range on some channel (for gates
// <= 0, |g| <= |G| on every row) takes another form instead: its staging
// forms only factors <= 1 (Kg, Qg, Kd = K e^{G - g}, e^{G}; no Kn), and all
// eight waves then form A and P (exact_chunk):
// - blocked, when each 16-row block's own gate sum is in range: the decay
//   between rows r and s (s <= r) splits at the cumulative gate rho_I before
//   r's row block I, e^{g_r - g_s} = e^{g_r - rho_I} e^{rho_I - g_s}, so the
//   tiles of row block I are matrix-core products of X_I = K_I e^{g - rho_I}
//   (and Q_I e^{g - rho_I}) with Y^(I) = K e^{rho_I - g} over the rows of
//   blocks 0..I: every factor is <= 1 except the second one inside block I,
//   which its gate sum bounds;
// - pairwise, otherwise: each entry summed over the channels with its own
//   factor (kda_exact.h).
// A row whose own |g| leaves the range while G does not (only possible with
// positive gates, outside the domain) gets NaN in its Qg entry: never
// finite and wrong.
constexpr float kSafeLog2 = 115.f;
constexpr int BRS = 40;      // bf16 stride of the blocked form's staged rows (32 channels)
static_assert(2 * C * BRS <= C * KS && (C + 32 * 3) * BRS <= C * KS,
              "X and Q X fit in one slot's Kg rows, the Y^(I) in its Qg rows");
static_assert((16 * DK + 4 * 256) * sizeof(float) <= C * KS * sizeof(uint16_t),
              "the group sums and B's diagonal blocks fit in Kn");
static_assert(NT == 16 * 32, "one 4 x 4 block of the chunk per thread");

// Byte-range views of one chunk of one head: row r of the chunk starts at
// r * row_bytes; the range ends with the last valid row's head segment.
struct ChunkView {
    __amdgpu_buffer_rsrc_t k, q, la, beta;
};

// With the front-end, la ranges over the bf16 gate pre-activations and
// beta over the bf16 beta pre-activations when they are given.
__device__ __forceinline__ ChunkView chunk_view(const bf16_t* k, const bf16_t* q,
                                                const float* log_alpha, const float* beta,
                                                int64_t c0, int len, int H, int h, int gate,
                                                const FrontEnd& fe) {
    const int64_t e0 = (c0 * H + h) * DK;               // first element of row 0
    const uint32_t span = static_cast<uint32_t>((len - 1) * H * DK + DK);
    const uint32_t hspan = static_cast<uint32_t>((len - 1) * H + 1);
    ChunkView cv;
    cv.k = rsrc(k + e0, 2u * span);
    cv.q = rsrc(q + e0, 2u * span);
    // gates: per key channel, or one per (token, head); none at all (a null
    // log_alpha) gives an empty range, where every load reads zero
    if (fe.gate_pre)
        cv.la = gate == kGateChannel ? rsrc(fe.gate_pre + e0, 2u * span)
                                     : rsrc(fe.gate_pre + c0 * H + h, 2u * hspan);
    else if (gate == kGateChannel)
        cv.la = rsrc(log_alpha + e0, 4u * span);
    else if (log_alpha)
        cv.la = rsrc(log_alpha + c0 * H + h, 4u * hspan);
    else
        cv.la = rsrc(log_alpha, 0u);
    cv.beta = fe.beta_pre ? rsrc(fe.beta_pre + c0 * H + h, 2u * hspan)
                          : rsrc(beta + c0 * H + h, 4u * hspan);
    return cv;
}

// The gate of row `row` of a chunk of `len` rows, channel pair (x, y), from
// what a stager or the strong-gate step loaded: fp32 gates as they are, or
// with the front-end's gate pre-activations (bf16, both channels in `raw`,
// or the row's one value) log_alpha = -scale softplus(x), zero past the
// sequence end (the loads read zero there, and softplus(0) is not).
template <int GATE>
__device__ __forceinline__ float2 front_gates(uint32_t raw, int row, int len, float scale) {
    if (row >= len) return make_float2(0.f, 0.f);
    if constexpr (GATE == kGateChannel)
        return make_float2(-scale * softplus_f32(lo_bf(raw)), -scale * softplus_f32(hi_bf(raw)));
    const float x = -scale * softplus_f32(lo_bf(raw));
    return make_float2(x, x);
}

// Stager registers: rows 16w .. 16w+15 of one chunk, key channels 2l, 2l+1
// for lane l, loaded one chunk ahead.
struct StageRegs {
    uint32_t k2[16], q2[16];
    u32x2 la[16];
};

// gate_pre: the front-end's bf16 gate pre-activations (raw bits in la[r][0],
// activated in place by front_rows before anything reads them).  In the
// front-end's instantiation the row offsets are formed at the load
// (opaque): hoisted, both gate layouts' 16 offsets would hold registers for
// the whole kernel.
template <int GATE, bool PRE>
__device__ __forceinline__ void load_rows_as(StageRegs& rg, const ChunkView& cv, int H, int w,
                                             int lane, bool opaque) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        int ro = 16 * w + r;
        if (opaque) asm volatile("" : "+v"(ro));
        const int off = ro * H * DK + 2 * lane;             // elements
        rg.k2[r] = ld32(cv.k, 2 * off);
        rg.q2[r] = ld32(cv.q, 2 * off);
        if constexpr (GATE == kGateChannel) {
            rg.la[r] = PRE ? u32x2{ld32(cv.la, 2 * off), 0u} : ld64(cv.la, 4 * off);
        } else {                                           // the row's scalar gate, both channels
            if constexpr (PRE) {
                rg.la[r] = u32x2{static_cast<uint32_t>(ld16(cv.la, 2 * ro * H)), 0u};
            } else {
                const uint32_t x = ld32(cv.la, 4 * ro * H);
                rg.la[r] = u32x2{x, x};
            }
        }
    }
}
template <int GATE, bool FRONT>
__device__ __forceinline__ void load_rows(StageRegs& rg, const ChunkView& cv, int H, int w,
                                          int lane, bool gate_pre) {
    if (FRONT && gate_pre) load_rows_as<GATE, true>(rg, cv, H, w, lane, FRONT);
    else load_rows_as<GATE, false>(rg, cv, H, w, lane, FRONT);
}

// The lane that DPP control CTRL selects (every row enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_from(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// x + y after v_permlane32_swap / v_permlane16_swap exchange the halves of
// the pair across lane bit 5 / bit 4: in lanes with that bit clear both
// terms are x (own and partner's), in the others both are y.
__device__ __forceinline__ float swap32_sum(float x, float y) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float swap16_sum(float x, float y) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sums over the 64 lanes of the wave of 16 values per lane (v[r]: row r),
// as a reduce-scatter: each step pairs lanes across one bit of the lane
// index, and each lane keeps half of its values (its partner the other
// half) and adds its partner's copy of that half -- lane bit 5 and bit 4
// through the permlane swaps, bit 3 and bit 2 through the row and half-row
// mirrors (each pairs across that bit), the last two bits summed by quad
// permutations.  Lane L ends with the total of row L / 4.  Every step is a
// VALU lane move; none goes through LDS.
__device__ __forceinline__ float wave_sum16_scatter(const float (&v)[16], int lane) {
    const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
    float w[8], x[4], y[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = swap32_sum(v[j], v[j + 8]);      // row j + 8 b5
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = swap16_sum(w[j], w[j + 4]);      // row 8 b5 + 4 b4 + j
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float keep = b3 ? x[j + 2] : x[j], send = b3 ? x[j] : x[j + 2];
        y[j] = keep + dpp_from<0x140>(send);          // row_mirror: lane 15 - p of the row
    }
    const float keep = b2 ? y[1] : y[0], send = b2 ? y[0] : y[1];
    float z = keep + dpp_from<0x141>(send);           // row_half_mirror: lane 7 - p of the 8
    z += dpp_from<0xb1>(z);                           // quad_perm [1, 0, 3, 2]
    z += dpp_from<0x4e>(z);                           // quad_perm [2, 3, 0, 1]
    return z;
}

// The front-end on a stager's loaded rows (before their gate sums): the
// gates from their pre-activations, in place, and the L2 norms of each
// row's k and q (reduced over the wave: a row is its 64 lanes' channel
// pairs) into nrm[0..1][row] as 1 / max(norm, eps).
template <int GATE>
__device__ __forceinline__ void front_rows(StageRegs& rg, float (*nrm)[C], const FrontEnd& fe,
                                           int w, int lane, int len) {
    // the loaded registers pass through an empty asm here, after the barrier
    // that precedes this step: the arithmetic below, which reads nothing
    // else from memory, would otherwise be scheduled right after the loads,
    // ahead of that barrier, and wait for them there (in the critical phase)
#pragma unroll
    for (int r = 0; r < 16; ++r)
        asm volatile("" : "+v"(rg.la[r][0]), "+v"(rg.la[r][1]), "+v"(rg.k2[r]), "+v"(rg.q2[r]));
    if (fe.gate_pre) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float2 a = front_gates<GATE>(rg.la[r][0], 16 * w + r, len, fe.gate_scale);
            rg.la[r] = u32x2{__float_as_uint(a.x), __float_as_uint(a.y)};
        }
    }
    if (fe.l2norm) {
        float vk[16], vq[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            vk[r] = lo_bf(rg.k2[r]) * lo_bf(rg.k2[r]) + hi_bf(rg.k2[r]) * hi_bf(rg.k2[r]);
            vq[r] = lo_bf(rg.q2[r]) * lo_bf(rg.q2[r]) + hi_bf(rg.q2[r]) * hi_bf(rg.q2[r]);
        }
        const float sk = wave_sum16_scatter(vk, lane), sq = wave_sum16_scatter(vq, lane);
        if ((lane & 3) == 0) {                        // lane L holds row L / 4
            nrm[0][16 * w + (lane >> 2)] = __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(sk), kFrontEps));
            nrm[1][16 * w + (lane >> 2)] = __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(sq), kFrontEps));
        }
    }
}

// Sum of the gates (in units of log2) over the 16 rows, per channel.
__device__ __forceinline__ float2 block_gate_sum(const StageRegs& rg) {
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        t0 = __builtin_fmaf(__uint_as_float(rg.la[r][0]), kLog2e, t0);
        t1 = __builtin_fmaf(__uint_as_float(rg.la[r][1]), kLog2e, t1);
    }
    return make_float2(t0, t1);
}

// Stage rows 16w .. 16w+15 into LDS slot b: cumulative gate, e^{+-g}, Kg,
// Qg, Kn, Kd^T (and e^{G} and the chunk's exact-form flag from stager 0).
// `tot` holds the four blocks' gate sums.  Rows past the end of the
// sequence hold zeros (they were read out of range), so they add nothing to
// the gate and contribute zero rows.  Every stager sees every channel's G,
// so all of them take the same branch.
// FRONT with l2norm: k and q of each row scaled by its 1 / norm (nrm[b]).
template <bool FRONT>
__device__ __forceinline__ void stage_rows(Smem& sm, int b, const StageRegs& rg,
                                           const float2* tot, int w, int lane, bool l2norm) {
    float run0 = 0.f, run1 = 0.f, G0 = 0.f, G1 = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const float2 t = tot[x * (DK / 2) + lane];
        if (x < w) { run0 += t.x; run1 += t.y; }
        G0 += t.x;
        G1 += t.y;
    }
    const bool exact = __ballot(!(fabsf(G0) <= kSafeLog2 && fabsf(G1) <= kSafeLog2)) != 0ull;
    const float gl0 = __builtin_amdgcn_exp2f(G0), gl1 = __builtin_amdgcn_exp2f(G1);
    if (w == 0) {
        *reinterpret_cast<float2*>(sm.gam[b] + 2 * lane) = make_float2(gl0, gl1);
        bool span = false;                      // a 16-row block's own sum beyond the range
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const float2 t = tot[x * (DK / 2) + lane];
            span |= !(fabsf(t.x) <= kSafeLog2 && fabsf(t.y) <= kSafeLog2);
        }
        const bool pairwise = __ballot(span) != 0ull;
        if (lane == 0) sm.xflag[b] = exact ? (pairwise ? 2 : 1) : 0;
    }
    float kd0[4], kd1[4];
    if (!exact) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * w + r;
            run0 = __builtin_fmaf(__uint_as_float(rg.la[r][0]), kLog2e, run0);   // g_row / ln 2
            run1 = __builtin_fmaf(__uint_as_float(rg.la[r][1]), kLog2e, run1);
            const bool wild = !(fabsf(run0) <= kSafeLog2 && fabsf(run1) <= kSafeLog2);
            const float u0 = __builtin_amdgcn_exp2f(run0), u1 = __builtin_amdgcn_exp2f(run1);
            const float w0 = __builtin_amdgcn_exp2f(-run0), w1 = __builtin_amdgcn_exp2f(-run1);
            float kx = lo_bf(rg.k2[r]), ky = hi_bf(rg.k2[r]);
            float qx = lo_bf(rg.q2[r]), qy = hi_bf(rg.q2[r]);
            if (FRONT && l2norm) {
                const float nk = sm.nrm[b][0][row], nq = sm.nrm[b][1][row];
                kx *= nk;
                ky *= nk;
                qx *= nq;
                qy *= nq;
            }
            const float n0 = kx * w0, n1 = ky * w1;
            *reinterpret_cast<uint32_t*>(sm.kg[b] + row * KS + 2 * lane) = pk(kx * u0, ky * u1);
            *reinterpret_cast<uint32_t*>(sm.qg[b] + row * KS + 2 * lane) =
                wild ? pk(nan, nan) : pk(qx * u0, qy * u1);
            *reinterpret_cast<uint32_t*>(sm.kn + row * KS + 2 * lane) = pk(n0, n1);
            kd0[r & 3] = n0 * gl0;
            kd1[r & 3] = n1 * gl1;
            if ((r & 3) == 3) {
                const int c0 = row - 3;
                *reinterpret_cast<u32x2*>(sm.kdt[b] + (2 * lane) * RS + c0) =
                    u32x2{pk(kd0[0], kd0[1]), pk(kd0[2], kd0[3])};
                *reinterpret_cast<u32x2*>(sm.kdt[b] + (2 * lane + 1) * RS + c0) =
                    u32x2{pk(kd1[0], kd1[1]), pk(kd1[2], kd1[3])};
            }
        }
    } else {
        // factors <= 1 only: e^{g}, e^{G - g}; A and P come from exact_chunk
        // (fully unrolled: the staged registers are indexed by row)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * w + r;
            run0 = __builtin_fmaf(__uint_as_float(rg.la[r][0]), kLog2e, run0);
            run1 = __builtin_fmaf(__uint_as_float(rg.la[r][1]), kLog2e, run1);
            const float u0 = __builtin_amdgcn_exp2f(run0), u1 = __builtin_amdgcn_exp2f(run1);
            const float d0 = __builtin_amdgcn_exp2f(G0 - run0), d1 = __builtin_amdgcn_exp2f(G1 - run1);
            float kx = lo_bf(rg.k2[r]), ky = hi_bf(rg.k2[r]);
            float qx = lo_bf(rg.q2[r]), qy = hi_bf(rg.q2[r]);
            if (FRONT && l2norm) {
                const float nk = sm.nrm[b][0][row], nq = sm.nrm[b][1][row];
                kx *= nk;
                ky *= nk;
                qx *= nq;
                qy *= nq;
            }
            *reinterpret_cast<uint32_t*>(sm.kg[b] + row * KS + 2 * lane) = pk(kx * u0, ky * u1);
            *reinterpret_cast<uint32_t*>(sm.qg[b] + row * KS + 2 * lane) = pk(qx * u0, qy * u1);
            kd0[r & 3] = kx * d0;
            kd1[r & 3] = ky * d1;
            if ((r & 3) == 3) {
                const int c0 = row - 3;
                *reinterpret_cast<u32x2*>(sm.kdt[b] + (2 * lane) * RS + c0) =
                    u32x2{pk(kd0[0], kd0[1]), pk(kd0[2], kd0[3])};
                *reinterpret_cast<u32x2*>(sm.kdt[b] + (2 * lane + 1) * RS + c0) =
                    u32x2{pk(kd1[0], kd1[1]), pk(kd1[2], kd1[3])};
            }
        }
    }
}

// 16x16 product of two 16-row bf16 blocks: D[m][n] = sum_c X[m][c] Y[n][c]
// (both operands in the same permuted K order)
__device__ __forceinline__ f32x4 row_product(const uint16_t* x, const uint16_t* y, int g, int ln) {
    const uint16_t* xr = x + ln * KS;
    const uint16_t* yr = y + ln * KS;
    u32x4 xf[4], yf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        xf[kk] = perm_row(xr, kk, g);
        yf[kk] = perm_row(yr, kk, g);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mma32(xf[kk], yf[kk], acc);
    return acc;
}

// The K-step fragments of one 16-row block of a [C][KS] operand, kept in
// registers so several products can share them.
struct BlockFrag {
    u32x4 f[4];
};
__device__ __forceinline__ BlockFrag block_frag(const uint16_t* rows, int blk, int g, int ln) {
    const uint16_t* r = rows + (16 * blk + ln) * KS;
    BlockFrag x;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) x.f[kk] = perm_row(r, kk, g);
    return x;
}
__device__ __forceinline__ f32x4 block_product(const BlockFrag& x, const BlockFrag& y) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mma32(x.f[kk], y.f[kk], acc);
    return acc;
}
// tile (I, J) of P (lower, diagonal included) and of -A (strictly lower)
__device__ __forceinline__ void put_p(Smem& sm, int b, int I, int J, const f32x4& acc, int g, int ln) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        sm.p[b][(16 * I + r) * RS + 16 * J + ln] = bf((I > J || r >= ln) ? acc[i] : 0.f);
    }
}
__device__ __forceinline__ void put_a(Smem& sm, int b, int I, int J, const f32x4& acc, int g, int ln) {
    uint16_t* blk = sm.an[b] + offdiag_index(I, J) * 16 * DS;
    const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta[b] + 16 * I + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) blk[(4 * g + i) * DS + ln] = bf(-bt[i] * acc[i]);
}

// One strictly-lower tile of A (which = 0) or any lower tile of P (which =
// 1) for LDS slot b.
__device__ __forceinline__ void tile_job(Smem& sm, int b, int which, int t, int g, int ln) {
    const int I = tile_row(t), J = tile_col(t);
    const f32x4 acc = row_product((which == 0 ? sm.kg[b] : sm.qg[b]) + 16 * I * KS,
                                  sm.kn + 16 * J * KS, g, ln);
    if (which == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            sm.p[b][(16 * I + r) * RS + 16 * J + ln] = bf((I > J || r >= ln) ? acc[i] : 0.f);
        }
        return;
    }
    uint16_t* blk = sm.an[b] + offdiag_index(I, J) * 16 * DS;
    const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta[b] + 16 * I + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) blk[(4 * g + i) * DS + ln] = bf(-bt[i] * acc[i]);
}

// Diagonal block I of A, N = strictly-lower(Diag(beta) Kg_I Kn_I^T), and the
// inverse (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0).
// With Y in the accumulator layout (lane (g, ln) holds Y[4g+i][ln]) passed
// as the A operand of a 16x16x16 product, the product sees Y^T; keeping both
// N and N^T lets every factor enter in the layout it is needed in.  The
// result is formed transposed, X^T = (I + N^2^T)(I + N^4^T)(I + N^8^T)(I -
// N^T), whose accumulator layout is exactly the A-operand layout of X.
__device__ __forceinline__ void diag_inverse(Smem& sm, int b, int I, const f32x4& a, const f32x4& at,
                                             int g, int ln);
__device__ __forceinline__ void diag_job(Smem& sm, int b, int I, int g, int ln) {
    const uint16_t* kgI = sm.kg[b] + 16 * I * KS;
    const uint16_t* knI = sm.kn + 16 * I * KS;
    const f32x4 a = row_product(kgI, knI, g, ln);    // (Kg_I Kn_I^T)[4g+i][ln]
    const f32x4 at = row_product(knI, kgI, g, ln);   // (Kg_I Kn_I^T)[ln][4g+i]
    diag_inverse(sm, b, I, a, at, g, ln);
}
// the inverse from a = (Kg_I Kn_I^T)[4g+i][ln] and at = (Kg_I Kn_I^T)[ln][4g+i]
__device__ __forceinline__ void diag_inverse(Smem& sm, int b, int I, const f32x4& a, const f32x4& at,
                                             int g, int ln) {
    const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta[b] + 16 * I + 4 * g);
    const float bl = sm.beta[b][16 * I + ln];
    f32x4 N, NT, eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        N[i] = (r > ln) ? bt[i] * a[i] : 0.f;       // N[r][ln]
        NT[i] = (ln > r) ? bl * at[i] : 0.f;        // N^T[r][ln] = N[ln][r]
        eye[i] = (r == ln) ? 1.f : 0.f;
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const u32x2 n_b = pack2(N), nt_b = pack2(NT);
    const f32x4 M2 = mma16(nt_b, n_b, zero);         // N N
    const f32x4 M2T = mma16(n_b, nt_b, zero);        // N^T N^T
    const u32x2 m2_b = pack2(M2), m2t_b = pack2(M2T);
    const f32x4 M4 = mma16(m2t_b, m2_b, zero);
    const f32x4 M4T = mma16(m2_b, m2t_b, zero);
    const f32x4 M8 = mma16(pack2(M4T), pack2(M4), zero);
    const f32x4 Z1 = mma16(pack2(eye + M8), pack2(eye - NT), zero);
    const f32x4 Z2 = mma16(pack2(eye + M4), pack2(Z1), zero);
    const f32x4 Z3 = mma16(pack2(eye + M2), pack2(Z2), zero);
    // lane (g, ln) holds X[ln][4g+i]: row ln, columns 4g..4g+3 of the inverse
    *reinterpret_cast<u32x2*>(sm.dinv[b] + (I * 16 + ln) * DS + 4 * g) = pack2(Z3);
}

}  // namespace

// FRONT: the fused input front-end (its own instantiation): q and k
// L2-normalised per row when fe.l2norm, gates from bf16 pre-activations
// (log_alpha = -fe.gate_scale softplus(x)) when fe.gate_pre, beta =
// sigmoid(y) from bf16 fe.beta_pre.  The stagers apply it to the rows they
// load, and the strong-gate step to the rows it reloads.
template <int TV, int GATE, bool FRONT>
__global__ __launch_bounds__(NT)
void prefill_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                         const bf16_t* __restrict__ v, const float* __restrict__ log_alpha,
                         const float* __restrict__ beta, const float* __restrict__ h0,
                         const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
                         int64_t groups, int R, int H, int DV, float scale,
                         bf16_t* __restrict__ o, float* __restrict__ hT,
                         float* __restrict__ snapshots, int snap_tokens, int snap_cap,
                         FrontEnd fe)
{
    if constexpr (!FRONT) fe = FrontEnd{};
    constexpr int NSLAB = TV / 16;                   // 16-column state slabs in the tile
    constexpr int NC = NSLAB < 4 ? NSLAB : 4;        // consumer waves
    constexpr int SPW = NSLAB / NC;                  // slabs per consumer wave (1 or 2)
    constexpr int NP = NW - NC;                      // producer waves
    static_assert(TV <= kMaxTileColumns && NSLAB == NC * SPW && SPW <= 2, "the slab map");
    static_assert(NP >= NSTAGE, "four stager waves");
    __shared__ Smem sm;

    int64_t pair;
    int tile;
    if (!prefill_map_block(blockIdx.x, groups, R, pair, tile)) return;
    const int tid = threadIdx.x;
    // the wave index is uniform across the wave: the roles below branch on it
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int h = static_cast<int>(pair % H);
    const int n = order[pair / H];
    const int64_t t_begin = cu[n];
    const int64_t t_end = cu[n + 1];
    const int nch = static_cast<int>((t_end - t_begin + C - 1) / C);
    const int j0 = tile * TV;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV + j0;

    auto chunk_start = [&](int m) { return t_begin + static_cast<int64_t>(m) * C; };
    auto chunk_len = [&](int m) { return static_cast<int>(min<int64_t>(C, t_end - chunk_start(m))); };

    for (int i = tid; i < C * RS; i += NT) reinterpret_cast<uint32_t*>(&sm.p[0][0])[i] = 0u;

    // P for LDS slot m & 1, with four consumers (the producers then take A
    // and the diagonal blocks):
    //   wave 0: P(0,0), P(3,0), P(3,3)    wave 1: P(1,0), P(1,1), P(3,1)
    //   wave 2: P(2,0), P(2,1)            wave 3: P(2,2), P(3,2)
    auto p_tiles4 = [](int m, int c, int g, int ln) __attribute__((always_inline)) {
        const int b = m & 1;
        const uint16_t* QG = sm.qg[b];
        const uint16_t* KN = sm.kn;
        if (c == 0) {
            const BlockFrag kn0 = block_frag(KN, 0, g, ln), qg3 = block_frag(QG, 3, g, ln);
            const BlockFrag qg0 = block_frag(QG, 0, g, ln);
            put_p(sm, b, 3, 0, block_product(qg3, kn0), g, ln);
            put_p(sm, b, 0, 0, block_product(qg0, kn0), g, ln);
            const BlockFrag kn3 = block_frag(KN, 3, g, ln);
            put_p(sm, b, 3, 3, block_product(qg3, kn3), g, ln);
        } else if (c == 1) {
            const BlockFrag kn0 = block_frag(KN, 0, g, ln), kn1 = block_frag(KN, 1, g, ln);
            const BlockFrag qg1 = block_frag(QG, 1, g, ln);
            put_p(sm, b, 1, 0, block_product(qg1, kn0), g, ln);
            put_p(sm, b, 1, 1, block_product(qg1, kn1), g, ln);
            const BlockFrag qg3 = block_frag(QG, 3, g, ln);
            put_p(sm, b, 3, 1, block_product(qg3, kn1), g, ln);
        } else if (c == 2) {
            const BlockFrag kn0 = block_frag(KN, 0, g, ln), kn1 = block_frag(KN, 1, g, ln);
            const BlockFrag qg2 = block_frag(QG, 2, g, ln);
            put_p(sm, b, 2, 0, block_product(qg2, kn0), g, ln);
            put_p(sm, b, 2, 1, block_product(qg2, kn1), g, ln);
        } else {
            const BlockFrag kn2 = block_frag(KN, 2, g, ln), qg2 = block_frag(QG, 2, g, ln);
            const BlockFrag qg3 = block_frag(QG, 3, g, ln);
            put_p(sm, b, 2, 2, block_product(qg2, kn2), g, ln);
            put_p(sm, b, 3, 2, block_product(qg3, kn2), g, ln);
        }
    };

    // A, P and the diagonal-block inverses of the chunk in LDS slot b beyond
    // the factored range, by all eight waves.  The chunk's k, q and gates are
    // read again (the stagers loaded them two chunks ago, so they are likely
    // still in L2) and staged 32 channels at a time in LDS that is dead at
    // this point: the other slot's Kg and Qg rows (the consumers read them in
    // the first phase only) and Kn (not formed for such a chunk).  Contains
    // barriers: every wave calls it, or none.
    auto exact_chunk = [](int b, ChunkView cv, int H, int tid, int wave, int g, int ln,
                          FrontEnd fe, int len) __attribute__((always_inline)) {
        if (sm.xflag[b] == 1) {
            // blocked form.  In each half, thread (rg, cg) loads rows
            // 4 rg .. +3, channels 4 cg + 2 half + {0, 1} (k, q as bf16
            // pairs), sums the gates within its row block (the 4-row group
            // sums go through LDS), and in round j stages channel
            // 4 cg + 2 half + j at column cg: X and Q X in the other slot's Kg
            // rows, Y^(I), I = 0..3 (16 (I + 1) rows each) in its Qg rows.
            // Wave w accumulates the 20 lower tiles w, w + 8, w + 16 (A, then
            // P) with one matrix-core step per round.
            uint16_t* bx = sm.kg[b ^ 1];
            uint16_t* bqx = bx + C * BRS;
            uint16_t* by = sm.qg[b ^ 1];
            float* gs = reinterpret_cast<float*>(sm.kn);     // [16][DK] 4-row group sums
            float* dt = gs + 16 * DK;                        // B's diagonal blocks, fp32
            // lane coordinates as opaque values: addresses formed from them
            // stay inside this rare branch instead of being hoisted out of
            // the chunk loop, where they would hold registers throughout
            int cg = tid & 31, rg = tid >> 5;
            asm volatile("" : "+v"(cg), "+v"(rg), "+v"(g), "+v"(ln), "+v"(wave));
            const int Ir = rg >> 2;
            f32x4 acc[3];
#pragma unroll
            for (int x = 0; x < 3; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int half = 0; half < 2; ++half) {
                uint32_t kw[4], qw[4];
                float gw[4][2];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int off = (4 * rg + i) * H * DK + 4 * cg + 2 * half;   // elements
                    kw[i] = ld32(cv.k, 2 * off);
                    qw[i] = ld32(cv.q, 2 * off);
                    if (FRONT && fe.gate_pre) {
                        const uint32_t raw = GATE == kGateChannel
                                                 ? ld32(cv.la, 2 * off)
                                                 : static_cast<uint32_t>(ld16(cv.la, 2 * (4 * rg + i) * H));
                        const float2 a = front_gates<GATE>(raw, 4 * rg + i, len, fe.gate_scale);
                        gw[i][0] = a.x;
                        gw[i][1] = a.y;
                    } else if constexpr (GATE == kGateChannel) {
                        const u32x2 l = ld64(cv.la, 4 * off);
                        gw[i][0] = __uint_as_float(l[0]);
                        gw[i][1] = __uint_as_float(l[1]);
                    } else {
                        gw[i][0] = gw[i][1] = __uint_as_float(ld32(cv.la, 4 * (4 * rg + i) * H));
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        gw[i][j] = __builtin_fmaf(gw[i][j], kLog2e, i > 0 ? gw[i - 1][j] : 0.f);
                *reinterpret_cast<float2*>(gs + rg * DK + 4 * cg + 2 * half) = make_float2(gw[3][0], gw[3][1]);
                __syncthreads();      // also: the last round's reads of the staged rows are done
                {
                    float b0 = 0.f, b1 = 0.f;           // the groups before this one in the block
                    for (int x = 4 * Ir; x < rg; ++x) {
                        const float2 t = *reinterpret_cast<const float2*>(gs + x * DK + 4 * cg + 2 * half);
                        b0 += t.x;
                        b1 += t.y;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        gw[i][0] += b0;
                        gw[i][1] += b1;
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // the gate sums of blocks 0..2 on this round's channel
                    const float2* tb = sm.tot[b] + 2 * cg + half;
                    float tt[3];
#pragma unroll
                    for (int x = 0; x < 3; ++x) tt[x] = j ? tb[x * (DK / 2)].y : tb[x * (DK / 2)].x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * rg + i;
                        float kx = j ? hi_bf(kw[i]) : lo_bf(kw[i]);
                        float qx = j ? hi_bf(qw[i]) : lo_bf(qw[i]);
                        if (FRONT && fe.l2norm) {
                            kx *= sm.nrm[b][0][r];
                            qx *= sm.nrm[b][1][r];
                        }
                        const float gr = gw[i][j];               // g_r - rho_Ir
                        const float f = __builtin_amdgcn_exp2f(gr);
                        bx[r * BRS + cg] = bf(kx * f);
                        bqx[r * BRS + cg] = bf(qx * f);
                        float e = -gr;                           // rho_I - g_r for I = Ir, Ir + 1, ..
#pragma unroll
                        for (int I = 0; I < 4; ++I) {
                            if (I < Ir) continue;
                            by[(8 * I * (I + 1) + r) * BRS + cg] = bf(kx * __builtin_amdgcn_exp2f(e));
                            if (I < 3) e += tt[I];
                        }
                    }
                    __syncthreads();
#pragma unroll
                    for (int x = 0; x < 3; ++x) {
                        const int t = wave + 8 * x;
                        if (t >= 20) continue;
                        const int tl = t < 10 ? t : t - 10;
                        const int I = tile_row(tl), J = tile_col(tl);
                        const uint16_t* xs = (t < 10 ? bx : bqx) + (16 * I + ln) * BRS + 8 * g;
                        const uint16_t* ys = by + (8 * I * (I + 1) + 16 * J + ln) * BRS + 8 * g;
                        acc[x] = mma32(*reinterpret_cast<const u32x4*>(xs),
                                       *reinterpret_cast<const u32x4*>(ys), acc[x]);
                    }
                    if (j == 0) __syncthreads();            // the staged rows are read
                }
            }
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int t = wave + 8 * x;
                if (t >= 20) continue;
                const int tl = t < 10 ? t : t - 10;
                const int I = tile_row(tl), J = tile_col(tl);
                if (t >= 10) {
                    put_p(sm, b, I, J, acc[x], g, ln);
                } else if (I > J) {
                    put_a(sm, b, I, J, acc[x], g, ln);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) dt[I * 256 + (4 * g + i) * 16 + ln] = acc[x][i];
                }
            }
            __syncthreads();
            if (wave < 4) {
                f32x4 av, at;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    av[i] = dt[wave * 256 + (4 * g + i) * 16 + ln];
                    at[i] = dt[wave * 256 + ln * 16 + 4 * g + i];
                }
                diag_inverse(sm, b, wave, av, at, g, ln);
            }
            return;
        }
        float* sk = reinterpret_cast<float*>(sm.kg[b ^ 1]);
        float* sq = reinterpret_cast<float*>(sm.qg[b ^ 1]);
        float* sg = reinterpret_cast<float*>(sm.kn);
        float* dt = sg + C * kExactXS;      // strictly lower entries of B's diagonal blocks
        float* gs = dt + 4 * 16 * 16;       // [16][32] gate sums of four-row groups
        const ExactUnit u = exact_unit(tid);
        float a[4][2], pp[4][2];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) a[x][y] = pp[x][y] = 0.f;
        const int c = tid & 31, r16 = tid >> 5;
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
            // channels 32j .. 32j + 31; this thread: channel c of rows 4 r16 .. +3
            float kk[4], qq[4], gg[4], run = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * r16 + i;
                const int off = row * H * DK + 32 * j + c;
                kk[i] = __uint_as_float(static_cast<uint32_t>(ld16(cv.k, 2 * off)) << 16);
                qq[i] = __uint_as_float(static_cast<uint32_t>(ld16(cv.q, 2 * off)) << 16);
                if (FRONT && fe.l2norm) {
                    kk[i] *= sm.nrm[b][0][row];
                    qq[i] *= sm.nrm[b][1][row];
                }
                if (FRONT && fe.gate_pre) {
                    // one channel (or the row's one gate): the low half
                    const uint32_t raw = ld16(cv.la, 2 * (GATE == kGateChannel ? off : row * H));
                    run += front_gates<kGateHead>(raw, row, len, fe.gate_scale).x;
                } else {
                    const uint32_t lb = GATE == kGateChannel ? ld32(cv.la, 4 * off) : ld32(cv.la, 4 * row * H);
                    run += __uint_as_float(lb);
                }
                gg[i] = run;
            }
            gs[r16 * 32 + c] = run;
            __syncthreads();
            float base = 0.f;
            for (int x = 0; x < r16; ++x) base += gs[x * 32 + c];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = (4 * r16 + i) * kExactXS + c;
                sk[e] = kk[i];
                sq[e] = qq[i];
                sg[e] = base + gg[i];
            }
            __syncthreads();
            exact_accumulate(u, sk, sq, sg, kLog2e, a, pp);
            __syncthreads();
        }
        exact_reduce(u, a, pp);
        if (exact_writer(u, tid)) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) {
                    const int r = 4 * u.bi + x, s2 = 2 * u.bj + y;
                    if (s2 <= r) sm.p[b][r * RS + s2] = bf(pp[x][y]);
                    if (s2 < r) {
                        const int I = r >> 4, J = s2 >> 4;
                        if (I > J)
                            sm.an[b][offdiag_index(I, J) * 16 * DS + (r & 15) * DS + (s2 & 15)] =
                                bf(-sm.beta[b][r] * a[x][y]);
                        else
                            dt[I * 256 + (r & 15) * 16 + (s2 & 15)] = a[x][y];
                    }
                }
        }
        __syncthreads();
        if (wave < 4) {
            f32x4 av, at;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = dt[wave * 256 + (4 * g + i) * 16 + ln];
                at[i] = dt[wave * 256 + ln * 16 + 4 * g + i];
            }
            diag_inverse(sm, b, wave, av, at, g, ln);
        }
    };
    auto view_of = [&](int m) {
        return chunk_view(k, q, log_alpha, beta, chunk_start(m), chunk_len(m), H, h, GATE, fe);
    };

    if (wave >= NC) {
        // ======================= producer waves =======================
        const int pw = wave - NC;
        // the producers' own copies of the lane coordinates: their LDS
        // addresses are then not shared with (and kept live for) the
        // consumer path
        int pg = g, pln = ln;
        asm volatile("" : "+v"(pg), "+v"(pln));
        const bool stager = pw < NSTAGE;
        StageRegs rg;
        uint32_t beta_next = 0u;
        auto prefetch = [&](int m) {
            if (!stager) return;
            const ChunkView cv = chunk_view(k, q, log_alpha, beta, chunk_start(m), chunk_len(m), H, h, GATE, fe);
            load_rows<GATE, FRONT>(rg, cv, H, pw, lane, FRONT && fe.gate_pre);
            if (pw == 0) {
                // the row offset formed here (an opaque lane index): hoisted,
                // it would hold a register for the whole kernel
                int lb = lane;
                asm volatile("" : "+v"(lb));
                beta_next = FRONT && fe.beta_pre ? static_cast<uint32_t>(ld16(cv.beta, 2 * lb * H))
                                                 : ld32(cv.beta, 4 * lb * H);
            }
        };
        auto totals = [&](int m) {
            if (!stager) return;
            if constexpr (FRONT) front_rows<GATE>(rg, sm.nrm[m & 1], fe, pw, lane, chunk_len(m));
            sm.tot[m & 1][pw * (DK / 2) + lane] = block_gate_sum(rg);
        };
        auto stage = [&](int m) {
            if (!stager) return;
            const int b = m & 1;
            stage_rows<FRONT>(sm, b, rg, sm.tot[b], pw, lane, fe.l2norm);
            if (pw == 0)
                sm.beta[b][lane] = FRONT && fe.beta_pre
                                       ? (lane < chunk_len(m) ? sigmoid_f32(lo_bf(beta_next)) : 0.f)
                                       : __uint_as_float(beta_next);
        };
        // A/P tile jobs, balanced greedily over the producers (weights: a
        // diagonal job with its inversion 3, a plain tile 1, the stagers'
        // gate sums 1); every wave computes the same assignment.
        int load[NW];
        for (int x = 0; x < NP; ++x) load[x] = (x < NSTAGE) ? 1 : 0;
        uint32_t mine = 0u;                          // bit j: job j is this wave's
        for (int j = 0; j < 20; ++j) {
            int best = 0;
            for (int x = 1; x < NP; ++x) if (load[x] < load[best]) best = x;
            load[best] += (j < 4) ? 3 : 1;
            if (best == pw) mine |= 1u << j;
        }
        // With four producers (and four consumers), the producers take A and
        // the diagonal blocks, each wave reusing the 16-row blocks it has
        // loaded and issuing its independent products ahead of the inversion
        // chain; the consumers take P (p_tiles4):
        //   wave 0: diagonal 0; A(3,0)
        //   wave 1: diagonal 1; A(1,0), A(3,1)
        //   wave 2: diagonal 2; A(2,0), A(2,1)
        //   wave 3: diagonal 3; A(3,2)
        auto tiles4 = [](int m, int pw, int g, int ln) __attribute__((always_inline)) {
            const int b = m & 1;
            const uint16_t* KG = sm.kg[b];
            const uint16_t* KN = sm.kn;
            if (pw == 0) {
                const BlockFrag kn0 = block_frag(KN, 0, g, ln), kg0 = block_frag(KG, 0, g, ln);
                const BlockFrag kg3 = block_frag(KG, 3, g, ln);
                const f32x4 a = block_product(kg0, kn0), at = block_product(kn0, kg0);
                put_a(sm, b, 3, 0, block_product(kg3, kn0), g, ln);
                diag_inverse(sm, b, 0, a, at, g, ln);
            } else if (pw == 1) {
                const BlockFrag kn1 = block_frag(KN, 1, g, ln), kg1 = block_frag(KG, 1, g, ln);
                const BlockFrag kn0 = block_frag(KN, 0, g, ln);
                const f32x4 a = block_product(kg1, kn1), at = block_product(kn1, kg1);
                put_a(sm, b, 1, 0, block_product(kg1, kn0), g, ln);
                const BlockFrag kg3 = block_frag(KG, 3, g, ln);
                put_a(sm, b, 3, 1, block_product(kg3, kn1), g, ln);
                diag_inverse(sm, b, 1, a, at, g, ln);
            } else if (pw == 2) {
                const BlockFrag kn2 = block_frag(KN, 2, g, ln), kg2 = block_frag(KG, 2, g, ln);
                const BlockFrag kn0 = block_frag(KN, 0, g, ln);
                const f32x4 a = block_product(kg2, kn2), at = block_product(kn2, kg2);
                put_a(sm, b, 2, 0, block_product(kg2, kn0), g, ln);
                const BlockFrag kn1 = block_frag(KN, 1, g, ln);
                put_a(sm, b, 2, 1, block_product(kg2, kn1), g, ln);
                diag_inverse(sm, b, 2, a, at, g, ln);
            } else {
                const BlockFrag kn3 = block_frag(KN, 3, g, ln), kg3 = block_frag(KG, 3, g, ln);
                const BlockFrag kn2 = block_frag(KN, 2, g, ln);
                const f32x4 a = block_product(kg3, kn3), at = block_product(kn3, kg3);
                put_a(sm, b, 3, 2, block_product(kg3, kn2), g, ln);
                diag_inverse(sm, b, 3, a, at, g, ln);
            }
        };
        auto tiles = [&](int m) {
            if (NP == 4) {
                tiles4(m, pw, pg, pln);
                return;
            }
            const int b = m & 1;
            // jobs 0..3: diagonal blocks; 4..9: strictly-lower A tiles 1,3,4,6,7,8;
            // 10..19: P tiles 0..9
            for (int j = 0; j < 20; ++j) {
                if (!((mine >> j) & 1u)) continue;
                if (j < 4) diag_job(sm, b, j, g, ln);
                else if (j < 10) {
                    const int o2 = j - 4;
                    tile_job(sm, b, 0, (o2 < 1) ? 1 : (o2 < 3) ? o2 + 2 : o2 + 3, g, ln);
                } else {
                    tile_job(sm, b, 1, j - 10, g, ln);
                }
            }
        };
        // same barrier sequence as the consumers: three in the prologue,
        // two per chunk
        if (nch > 0) {
            prefetch(0);
            totals(0);
            __syncthreads();
            stage(0);
            if (nch > 1) prefetch(1);
            __syncthreads();
            const bool x0 = sm.xflag[0] != 0;
            if (!x0) tiles(0);
            if (nch > 1) totals(1);
            if (x0) exact_chunk(0, view_of(0), H, tid, wave, g, ln, fe, chunk_len(0));
            __syncthreads();
        }
        for (int ci = 0; ci < nch; ++ci) {
            if (ci + 1 < nch) {
                stage(ci + 1);
                if (ci + 2 < nch) prefetch(ci + 2);
            }
            __syncthreads();
            const bool xn = ci + 1 < nch && sm.xflag[(ci + 1) & 1] != 0;
            if (ci + 1 < nch && !xn) tiles(ci + 1);
            if (ci + 2 < nch) totals(ci + 2);
            if (xn) exact_chunk((ci + 1) & 1, view_of(ci + 1), H, tid, wave, g, ln, fe, chunk_len(ci + 1));
            __syncthreads();
        }
        return;
    }

    // ======================= consumer waves =======================
    // SPW fp32 state slabs in the accumulator layout:
    // S[s][m][i] = state[c = 16m + 4g + i][j = (wave SPW + s) 16 + ln]
    f32x4 S[SPW][8];
    int jc[SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        jc[s] = (wave * SPW + s) * 16 + ln;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[s][m][i] = h0 ? h0[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc[s]] : 0.f;
    }
    const int vrow = H * DV;                         // elements between token rows
    auto v_view = [&](int m) {
        const int len = chunk_len(m);
        return rsrc(v + (chunk_start(m) * H + h) * DV + j0,
                    2u * static_cast<uint32_t>((len - 1) * vrow + TV));
    };
    // V and O move in 8-byte row pieces: lane (g, ln) of a 16 x 16 block
    // holds row ln, columns 4g .. 4g+3 -- the A-operand layout of that block.
    // One 16x16x16 product with the identity turns it into the accumulator
    // layout (rows 4g + i, column ln) and back; bf16 values times 1 and 0
    // summed in fp32 are exact.
    const int slab_col = wave * SPW * 16 + 4 * g;   // first column of the lane's piece, slab 0
    u32x2 ident;
    {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = (4 * g + i == ln) ? 1.f : 0.f;
        ident = u32x2{pk(e[0], e[1]), pk(e[2], e[3])};
    }
    u32x2 vnext[SPW][4];                             // V of the next chunk, block I, slab s
    auto load_v = [&](int m) {
        const __amdgpu_buffer_rsrc_t rv = v_view(m);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const int off = 2 * ((16 * I + ln) * vrow + slab_col);
#pragma unroll
            for (int s = 0; s < SPW; ++s) vnext[s][I] = ld64(rv, off + 32 * s);
        }
    };

    if (nch > 0) {
        load_v(0);
        __syncthreads();
        __syncthreads();
        if (sm.xflag[0] != 0)
            exact_chunk(0, view_of(0), H, tid, wave, g, ln, fe, chunk_len(0));
        else if (NP == 4)
            p_tiles4(0, wave, g, ln);
        __syncthreads();
    }
    int snap_left = snapshots ? snap_tokens / C : 0;
    for (int ci = 0; ci < nch; ++ci) {
        const int b = ci & 1;
        const int len = chunk_len(ci);

        // ---------------- phase 1: Y = Kg S0, X, E ----------------
        // row block by row block: Y_I = Kg_I S0, X_I = Diag(beta_I)(V_I - Y_I),
        // then (I + A) E = X by block forward substitution,
        //   E_I = (I + A_II)^{-1} (X_I - sum_{J<I} A_IJ E_J)
        u32x4 sb[SPW][4];
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sb[s][kk] = pack4(S[s][2 * kk], S[s][2 * kk + 1]);
        u32x2 an_f[6], di_f[4];
#pragma unroll
        for (int x = 0; x < 6; ++x)
            an_f[x] = *reinterpret_cast<const u32x2*>(sm.an[b] + (x * 16 + ln) * DS + 4 * g);
#pragma unroll
        for (int I = 0; I < 4; ++I)
            di_f[I] = *reinterpret_cast<const u32x2*>(sm.dinv[b] + (I * 16 + ln) * DS + 4 * g);
        u32x2 eb[SPW][4];
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const uint16_t* row = sm.kg[b] + (16 * I + ln) * KS;
            u32x4 fr[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fr[kk] = perm_row(row, kk, g);
            const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta[b] + 16 * I + 4 * g);
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mma32(fr[kk], sb[s][kk], acc);
                const f32x4 vv = mma16(vnext[s][I], ident, zero);   // V rows 4g + i, column ln
                f32x4 z;
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = bt[i] * (vv[i] - acc[i]);
#pragma unroll
                for (int J = 0; J < I; ++J) z = mma16(an_f[offdiag_index(I, J)], eb[s][J], z);
                eb[s][I] = pack2(mma16(di_f[I], pack2(z), zero));
            }
        }
        if (ci + 1 < nch) load_v(ci + 1);

        // O: the start state's bf16 copy dies here, before the barrier
        const __amdgpu_buffer_rsrc_t ro = rsrc(o + (chunk_start(ci) * H + h) * DV + j0,
                                               2u * static_cast<uint32_t>((len - 1) * vrow + TV));
        u32x4 e01[SPW], e23[SPW];
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            e01[s] = cat(eb[s][0], eb[s][1]);
            e23[s] = cat(eb[s][2], eb[s][3]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            // O = scale (Qg S0 + P E); rows past the end are dropped by the range check
            const uint16_t* qrow = sm.qg[b] + (16 * I + ln) * KS;
            const uint16_t* prow = sm.p[b] + (16 * I + ln) * RS;
            u32x4 fr[6];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fr[kk] = perm_row(qrow, kk, g);
            fr[4] = perm_row(prow, 0, g);
            if (I >= 2) fr[5] = perm_row(prow, 1, g);
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mma32(fr[kk], sb[s][kk], acc);
                acc = mma32(fr[4], e01[s], acc);
                if (I >= 2) acc = mma32(fr[5], e23[s], acc);
                // bf16 (round to nearest even), then to row pieces and out
                const f32x4 t = mma16(pack2(scale * acc), ident, zero);
                st64(ro, 2 * ((16 * I + ln) * vrow + slab_col) + 32 * s, pack2(t));
            }
        }
        __syncthreads();

        // ---------------- phase 2: the state update ----------------
        // S = Diag(e^{G}) S0 + Kd^T E
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint16_t* krow = sm.kdt[b] + (16 * m + ln) * RS;
            const u32x4 f0 = perm_row(krow, 0, g), f1 = perm_row(krow, 1, g);
            const f32x4 gm = *reinterpret_cast<const f32x4*>(sm.gam[b] + 16 * m + 4 * g);
#pragma unroll
            for (int s = 0; s < SPW; ++s) S[s][m] = mma32(f1, e23[s], mma32(f0, e01[s], gm * S[s][m]));
        }
        // a snapshot after every snap_tokens / C chunks (a countdown: one
        // decrement per chunk on the serial path)
        const int js = snapshots && --snap_left == 0
                           ? (snap_left = snap_tokens / C, (ci + 1) / (snap_tokens / C) - 1) : -1;
        if (js >= 0 && js < snap_cap && len == C) {      // only a full chunk ends on a boundary
            float* dst = snapshot_at(snapshots, snap_cap, H, static_cast<int64_t>(DK) * DV, n, js, h) + j0;
            // the lane's part of the offsets, formed here: hoisted out of
            // the chunk loop, 64 per-element addresses would stay live
            int lp = 4 * g * DV + jc[0];
            asm volatile("" : "+v"(lp));
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int m = 0; m < 8; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[static_cast<int64_t>(16 * m + i) * DV + lp + 16 * s] = S[s][m][i];
        }
        if (ci + 1 < nch) {
            if (sm.xflag[(ci + 1) & 1] != 0)
                exact_chunk((ci + 1) & 1, view_of(ci + 1), H, tid, wave, g, ln, fe, chunk_len(ci + 1));
            else if (NP == 4)
                p_tiles4(ci + 1, wave, g, ln);
        }
        __syncthreads();
    }

    if (hT) {
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hT[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc[s]] = S[s][m][i];
    }
}

template <int TV, int GATE, bool FRONT>
static hipError_t launch_mfma_g(const PrefillArgs& a, int R, hipStream_t stream) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    const int64_t blocks = prefill_grid_blocks(groups, R);
    hipLaunchKernelGGL((prefill_mfma_kernel<TV, GATE, FRONT>), dim3(static_cast<unsigned>(blocks)), dim3(NT),
                       0, stream, static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.log_alpha, a.beta, a.h0, a.cu_seqlens,
                       a.order, groups, R, a.H, a.d_v, a.scale, static_cast<bf16_t*>(a.o), a.hT,
                       a.snapshots, a.snap_tokens, a.snap_cap, a.fe);
    return hipGetLastError();
}

// a per-head gate and no gate share one instantiation (no gate reads an
// empty range: zeros); the front-end has instantiations of its own
template <int TV>
static hipError_t launch_mfma_t(const PrefillArgs& a, int R, hipStream_t stream) {
    if (a.fe.active())
        return a.gate == kGateChannel ? launch_mfma_g<TV, kGateChannel, true>(a, R, stream)
                                      : launch_mfma_g<TV, kGateHead, true>(a, R, stream);
    return a.gate == kGateChannel ? launch_mfma_g<TV, kGateChannel, false>(a, R, stream)
                                  : launch_mfma_g<TV, kGateHead, false>(a, R, stream);
}

bool mfma_supported(const PrefillArgs& a) {
    return !a.dtype_f32 && a.d_k == DK && a.H <= kMaxHeads;
}

// Value tiles per (sequence, head): tiles of at most 64 columns (one slab
// per consumer wave), and enough work-groups to cover the 256 compute
// units, but tiles no narrower than 16 columns.
int mfma_value_tiles(const PrefillArgs& a) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    int R = a.d_v > kMaxTileColumns ? a.d_v / kMaxTileColumns : 1;
    while (R < a.d_v / 16 && groups * R < 256) R *= 2;
    return R;
}

bool mfma_tiles_ok(int d_v, int R) {
    return R > 0 && (R & (R - 1)) == 0 && d_v % R == 0 && d_v / R >= 16 &&
           d_v / R <= kMaxTileColumns;
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
