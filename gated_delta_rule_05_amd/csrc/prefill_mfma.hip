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
constexpr int RS = C + 8;    // bf16 row stride of Kd^T and P
constexpr int DS = 20;       // bf16 row stride of 16x16 blocks (-A off-diagonal, inverses)
constexpr int NSTAGE = 4;    // stager waves, 16 rows of each chunk apiece
constexpr int kMaxTileColumns = 64;  // one 16-column slab per consumer wave
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
};

// Byte-range views of one chunk of one head: row r of the chunk starts at
// r * row_bytes; the range ends with the last valid row's head segment.
struct ChunkView {
    __amdgpu_buffer_rsrc_t k, q, la, beta;
};

__device__ __forceinline__ ChunkView chunk_view(const bf16_t* k, const bf16_t* q,
                                                const float* log_alpha, const float* beta,
                                                int64_t c0, int len, int H, int h, int gate) {
    const int64_t e0 = (c0 * H + h) * DK;               // first element of row 0
    const uint32_t span = static_cast<uint32_t>((len - 1) * H * DK + DK);
    ChunkView cv;
    cv.k = rsrc(k + e0, 2u * span);
    cv.q = rsrc(q + e0, 2u * span);
    // gates: per key channel, or one per (token, head); none at all (a null
    // log_alpha) gives an empty range, where every load reads zero
    if (gate == kGateChannel)
        cv.la = rsrc(log_alpha + e0, 4u * span);
    else if (log_alpha)
        cv.la = rsrc(log_alpha + c0 * H + h, 4u * static_cast<uint32_t>((len - 1) * H + 1));
    else
        cv.la = rsrc(log_alpha, 0u);
    cv.beta = rsrc(beta + c0 * H + h, 4u * static_cast<uint32_t>((len - 1) * H + 1));
    return cv;
}

// Stager registers: rows 16w .. 16w+15 of one chunk, key channels 2l, 2l+1
// for lane l, loaded one chunk ahead.
struct StageRegs {
    uint32_t k2[16], q2[16];
    u32x2 la[16];
};

template <int GATE>
__device__ __forceinline__ void load_rows(StageRegs& rg, const ChunkView& cv, int H, int w,
                                          int lane) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int off = (16 * w + r) * H * DK + 2 * lane;   // elements
        rg.k2[r] = ld32(cv.k, 2 * off);
        rg.q2[r] = ld32(cv.q, 2 * off);
        if constexpr (GATE == kGateChannel) {
            rg.la[r] = ld64(cv.la, 4 * off);
        } else {                                           // the row's scalar gate, both channels
            const uint32_t x = ld32(cv.la, 4 * (16 * w + r) * H);
            rg.la[r] = u32x2{x, x};
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
// Qg, Kn, Kd^T (and e^{G} from stager 0).  `tot` holds the four blocks'
// gate sums.  Rows past the end of the sequence hold zeros (they were read
// out of range), so they add nothing to the gate and contribute zero rows.
__device__ __forceinline__ void stage_rows(Smem& sm, int b, const StageRegs& rg,
                                           const float2* tot, int w, int lane) {
    float run0 = 0.f, run1 = 0.f, G0 = 0.f, G1 = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const float2 t = tot[x * (DK / 2) + lane];
        if (x < w) { run0 += t.x; run1 += t.y; }
        G0 += t.x;
        G1 += t.y;
    }
    const float gl0 = __builtin_amdgcn_exp2f(G0), gl1 = __builtin_amdgcn_exp2f(G1);
    if (w == 0) *reinterpret_cast<float2*>(sm.gam[b] + 2 * lane) = make_float2(gl0, gl1);
    float kd0[4], kd1[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * w + r;
        run0 = __builtin_fmaf(__uint_as_float(rg.la[r][0]), kLog2e, run0);   // g_row / ln 2
        run1 = __builtin_fmaf(__uint_as_float(rg.la[r][1]), kLog2e, run1);
        const float u0 = __builtin_amdgcn_exp2f(run0), u1 = __builtin_amdgcn_exp2f(run1);
        const float w0 = __builtin_amdgcn_exp2f(-run0), w1 = __builtin_amdgcn_exp2f(-run1);
        const float kx = lo_bf(rg.k2[r]), ky = hi_bf(rg.k2[r]);
        const float qx = lo_bf(rg.q2[r]), qy = hi_bf(rg.q2[r]);
        const float n0 = kx * w0, n1 = ky * w1;
        *reinterpret_cast<uint32_t*>(sm.kg[b] + row * KS + 2 * lane) = pk(kx * u0, ky * u1);
        *reinterpret_cast<uint32_t*>(sm.qg[b] + row * KS + 2 * lane) = pk(qx * u0, qy * u1);
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
__device__ __forceinline__ void diag_job(Smem& sm, int b, int I, int g, int ln) {
    const uint16_t* kgI = sm.kg[b] + 16 * I * KS;
    const uint16_t* knI = sm.kn + 16 * I * KS;
    const f32x4 a = row_product(kgI, knI, g, ln);    // (Kg_I Kn_I^T)[4g+i][ln]
    const f32x4 at = row_product(knI, kgI, g, ln);   // (Kg_I Kn_I^T)[ln][4g+i]
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

template <int TV, int GATE>
__global__ __launch_bounds__(NT)
void prefill_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                         const bf16_t* __restrict__ v, const float* __restrict__ log_alpha,
                         const float* __restrict__ beta, const float* __restrict__ h0,
                         const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
                         int64_t groups, int R, int H, int DV, float scale,
                         bf16_t* __restrict__ o, float* __restrict__ hT,
                         float* __restrict__ snapshots, int snap_tokens, int snap_cap)
{
    constexpr int NSLAB = TV / 16;                   // 16-column state slabs in the tile
    constexpr int NC = NSLAB < 4 ? NSLAB : 4;        // consumer waves, one slab each
    constexpr int NP = NW - NC;                      // producer waves
    static_assert(TV <= kMaxTileColumns && NSLAB == NC, "one slab per consumer wave");
    static_assert(NP >= NSTAGE, "four stager waves");
    __shared__ Smem sm;

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
    const int nch = static_cast<int>((t_end - t_begin + C - 1) / C);
    const int j0 = tile * TV;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV + j0;

    auto chunk_start = [&](int m) { return t_begin + static_cast<int64_t>(m) * C; };
    auto chunk_len = [&](int m) { return static_cast<int>(min<int64_t>(C, t_end - chunk_start(m))); };

    for (int i = tid; i < C * RS; i += NT) reinterpret_cast<uint32_t*>(&sm.p[0][0])[i] = 0u;

    if (wave >= NC) {
        // ======================= producer waves =======================
        const int pw = wave - NC;
        const bool stager = pw < NSTAGE;
        StageRegs rg;
        uint32_t beta_next = 0u;
        auto prefetch = [&](int m) {
            if (!stager) return;
            const ChunkView cv = chunk_view(k, q, log_alpha, beta, chunk_start(m), chunk_len(m), H, h, GATE);
            load_rows<GATE>(rg, cv, H, pw, lane);
            if (pw == 0) beta_next = ld32(cv.beta, 4 * lane * H);
        };
        auto totals = [&](int m) {
            if (stager) sm.tot[m & 1][pw * (DK / 2) + lane] = block_gate_sum(rg);
        };
        auto stage = [&](int m) {
            if (!stager) return;
            const int b = m & 1;
            stage_rows(sm, b, rg, sm.tot[b], pw, lane);
            if (pw == 0) sm.beta[b][lane] = __uint_as_float(beta_next);
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
        auto tiles = [&](int m) {
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
            tiles(0);
            if (nch > 1) totals(1);
            __syncthreads();
        }
        for (int ci = 0; ci < nch; ++ci) {
            if (ci + 1 < nch) {
                stage(ci + 1);
                if (ci + 2 < nch) prefetch(ci + 2);
            }
            __syncthreads();
            if (ci + 1 < nch) tiles(ci + 1);
            if (ci + 2 < nch) totals(ci + 2);
            __syncthreads();
        }
        return;
    }

    // ======================= consumer waves =======================
    // fp32 state slab in the accumulator layout:
    // S[m][i] = state[c = 16m + 4g + i][j = wave * 16 + ln]
    const int jc = wave * 16 + ln;
    f32x4 S[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[m][i] = h0 ? h0[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc] : 0.f;
    const int vrow = H * DV;                         // elements between token rows
    auto v_view = [&](int m) {
        const int len = chunk_len(m);
        return rsrc(v + (chunk_start(m) * H + h) * DV + j0,
                    2u * static_cast<uint32_t>((len - 1) * vrow + TV));
    };
    uint16_t vnext[16];                              // V of the next chunk, rows 16I + 4g + i
    auto load_v = [&](int m) {
        const __amdgpu_buffer_rsrc_t rv = v_view(m);
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vnext[4 * I + i] = ld16(rv, 2 * ((16 * I + 4 * g + i) * vrow + jc));
    };

    if (nch > 0) {
        load_v(0);
        __syncthreads();
        __syncthreads();
        __syncthreads();
    }
    int snap_left = snapshots ? snap_tokens / C : 0;
    for (int ci = 0; ci < nch; ++ci) {
        const int b = ci & 1;
        const int len = chunk_len(ci);

        // ---------------- phase 1: Y = Kg S0, X, E ----------------
        u32x4 sb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sb[kk] = pack4(S[2 * kk], S[2 * kk + 1]);
        f32x4 X[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const uint16_t* row = sm.kg[b] + (16 * I + ln) * KS;
            u32x4 fr[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fr[kk] = perm_row(row, kk, g);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mma32(fr[kk], sb[kk], acc);
            const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta[b] + 16 * I + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X[I][i] = bt[i] * (__uint_as_float(static_cast<uint32_t>(vnext[4 * I + i]) << 16) - acc[i]);
        }
        if (ci + 1 < nch) load_v(ci + 1);
        // (I + A) E = X by block forward substitution
        u32x2 an_f[6], di_f[4];
#pragma unroll
        for (int x = 0; x < 6; ++x)
            an_f[x] = *reinterpret_cast<const u32x2*>(sm.an[b] + (x * 16 + ln) * DS + 4 * g);
#pragma unroll
        for (int I = 0; I < 4; ++I)
            di_f[I] = *reinterpret_cast<const u32x2*>(sm.dinv[b] + (I * 16 + ln) * DS + 4 * g);
        u32x2 eb[4];
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 z = X[I];
#pragma unroll
            for (int J = 0; J < I; ++J) z = mma16(an_f[offdiag_index(I, J)], eb[J], z);
            eb[I] = pack2(mma16(di_f[I], pack2(z), zero));
        }
        __syncthreads();

        // ---------------- phase 2: O and the state update ----------------
        const __amdgpu_buffer_rsrc_t ro = rsrc(o + (chunk_start(ci) * H + h) * DV + j0,
                                               2u * static_cast<uint32_t>((len - 1) * vrow + TV));
        const u32x4 e01 = cat(eb[0], eb[1]), e23 = cat(eb[2], eb[3]);
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
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mma32(fr[kk], sb[kk], acc);
            acc = mma32(fr[4], e01, acc);
            if (I >= 2) acc = mma32(fr[5], e23, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st16(ro, 2 * ((16 * I + 4 * g + i) * vrow + jc), bf(scale * acc[i]));
        }
        // S = Diag(e^{G}) S0 + Kd^T E
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint16_t* krow = sm.kdt[b] + (16 * m + ln) * RS;
            const u32x4 f0 = perm_row(krow, 0, g), f1 = perm_row(krow, 1, g);
            const f32x4 gm = *reinterpret_cast<const f32x4*>(sm.gam[b] + 16 * m + 4 * g);
            S[m] = mma32(f1, e23, mma32(f0, e01, gm * S[m]));
        }
        // a snapshot after every snap_tokens / C chunks (a countdown: one
        // decrement per chunk on the serial path)
        const int js = snapshots && --snap_left == 0
                           ? (snap_left = snap_tokens / C, (ci + 1) / (snap_tokens / C) - 1) : -1;
        if (js >= 0 && js < snap_cap && len == C) {      // only a full chunk ends on a boundary
            float* dst = snapshot_at(snapshots, snap_cap, H, static_cast<int64_t>(DK) * DV, n, js, h) + j0 + jc;
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[static_cast<int64_t>(16 * m + 4 * g + i) * DV] = S[m][i];
        }
        __syncthreads();
    }

    if (hT) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hT[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc] = S[m][i];
    }
}

template <int TV, int GATE>
static hipError_t launch_mfma_g(const PrefillArgs& a, int R, hipStream_t stream) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    const int64_t blocks = prefill_grid_blocks(groups, R);
    hipLaunchKernelGGL((prefill_mfma_kernel<TV, GATE>), dim3(static_cast<unsigned>(blocks)), dim3(NT),
                       0, stream, static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.log_alpha, a.beta, a.h0, a.cu_seqlens,
                       a.order, groups, R, a.H, a.d_v, a.scale, static_cast<bf16_t*>(a.o), a.hT,
                       a.snapshots, a.snap_tokens, a.snap_cap);
    return hipGetLastError();
}

// a per-head gate and no gate share one instantiation (no gate reads an
// empty range: zeros)
template <int TV>
static hipError_t launch_mfma_t(const PrefillArgs& a, int R, hipStream_t stream) {
    return a.gate == kGateChannel ? launch_mfma_g<TV, kGateChannel>(a, R, stream)
                                  : launch_mfma_g<TV, kGateHead>(a, R, stream);
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
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
