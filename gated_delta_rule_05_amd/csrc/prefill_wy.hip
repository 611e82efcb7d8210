// prefill_wy.hip -- two-pass chunked KDA prefill on gfx950 matrix cores
// (bf16 operands, fp32 accumulation, fp32 state), d_k = 128, chunks of 64
// tokens.  Meant for batches with few (sequence, head) pairs, where the
// serial walk over chunks, not the total work, sets the time.
//
// Per chunk of C = 64 tokens with start state S0 (d_k x d_v, fp32), per key
// channel c (the chunked form of the per-token recurrence; the pages only
// say it is evaluated blockwise, with a diagonal-plus-low-rank transition):
//   g_r  = sum_{s<=r} log_alpha_s,  G = g_last
//   Kg   = K * e^{g},  Qg = Q * e^{g},  Kn = K * e^{-g},  Kd = K * e^{G-g}
//   A    = strictly-lower(Diag(beta) Kg Kn^T)
//   T    = (I + A)^{-1} Diag(beta)          (UT transform of the delta rule)
//   W    = T Kg,  U = T V,  P = lower(Qg Kn^T)
//   E    = U - W S0                          the chunk's delta errors
//   O    = scale (Qg S0 + P E)
//   S    = Diag(e^{G}) S0 + Kd^T E
// The factors of the chunked form split at the chunk start, so a row's
// factors depend only on the gates up to that row: an output never depends,
// even in rounding, on tokens after it.
//
// Pass 1, the prep kernel: one work-group per (chunk, head), all chunks at
// once.  It computes everything that does not depend on the state -- W, U,
// Qg, Kd^T, P and e^{G} -- and writes them to a workspace slot already in
// the MFMA operand layouts (kda_mfma.h) that pass 2 feeds to the matrix
// cores, so pass 2 copies them without any rearranging.  T comes from the
// inverses of the 16x16 diagonal blocks of I + A (on MFMA, from (I + N)^{-1}
// = (I - N)(I + N^2)(I + N^4)(I + N^8) for the nilpotent N = A_II) and a
// block forward substitution for the blocks below them.
// Pass 2, the carry kernel: one work-group per (sequence, head, value tile)
// walks the chunks in order with its fp32 state slabs in registers.  Per
// chunk it needs two products on the serial path (W S0, then Kd^T E), done
// by a state wave per 16-column slab, and one off it (O), done one chunk
// later by an output wave from the state wave's handover of S0 and E.
// Loader waves copy the next chunk's slot into the other half of a double
// buffer in LDS, their global loads four chunks ahead.
// The host alternates the passes over blocks of chunks, so the workspace
// holds a bounded block of slots (and stays mostly cache-resident) while
// the state is carried between blocks through hT (or a workspace copy).
#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_exact.h"
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_sched.h"

namespace kda {
namespace {

constexpr int C = 64;          // tokens per chunk
constexpr int DK = 128;        // key channels
constexpr int kMaxHeads = 16384;   // keeps every chunk-relative byte offset in 31 bits

// ---- workspace slot of one (chunk, head), bytes
constexpr int kFrag = 1024;                 // one MFMA operand: 64 lanes x 16 B
constexpr int kFragQ = 0;                   // Qg:    [I 4][kk 4] A operands
constexpr int kFragP = 16;                  // P:     (I,kk) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
constexpr int kFragW = 22;                  // -W:    [I 4][kk 4] A operands (negated: E = U + (-W) S0)
constexpr int kFragK = 38;                  // Kd^T:  [m 8][kk 2] A operands
constexpr int kNumFrag = 54;
// the carry's output waves read Qg and P straight into registers; the rest
// (W, Kd^T, e^{G}, U) is staged through LDS, from this byte on
constexpr int kStageOff = kFragW * kFrag;
constexpr int kOffGam = kNumFrag * kFrag;   // e^{G}: 128 fp32
constexpr int kOffU = kOffGam + 512;        // U: [slab d_v/16][I 4][64 lanes][4 bf16]
constexpr int kSlabBytes = 4 * 64 * 8;      // U of one 16-column slab
__host__ __device__ constexpr int slot_bytes(int dv) { return kOffU + 128 * dv; }
static_assert(kOffU % 256 == 0 && kStageOff % 256 == 0, "slots stay 256-byte aligned");

__device__ __forceinline__ int p_frag(int I, int kk) { return I < 2 ? I : 2 * I - 2 + kk; }

// position of index x of a row stored in fragment order: in each 32-wide
// block, K-step group g reads 8 consecutive entries, x = 4g + j and
// 16 + 4g + j (j < 4)
__device__ __forceinline__ int fpos(int x) {
    const int y = x & 31;
    return (x & ~31) + 8 * ((y & 15) >> 2) + 4 * (y >> 4) + (y & 3);
}

// ===================================================================
// pass 1: prep
// ===================================================================
constexpr int PT = 512;        // threads (8 waves)
constexpr int TS = DK + 8;     // bf16 stride of token rows (272 B: conflict-free 16-byte reads)
constexpr int CS = C + 8;      // bf16 stride of channel rows (144 B)
constexpr int BS = 20;         // bf16 stride of 16x16 blocks

struct alignas(16) PrepSmem {
    uint16_t tok[3][C * TS];   // Kg, Kn, Qg: token rows, channels in fragment order
    float beta[C];
    float glog[DK];            // G / ln 2
    float rho[3][DK];          // cumulative gate before row block 1, 2, 3 (log2 units)
    int exact;                 // nonzero: A and P outside the factored form
    int pairwise;              // nonzero: ... and a 16-row block spans beyond it too
};
// 53 KB: three work-groups fit in one CU's LDS.  Reuse of the token rows:
// - tok[0] first holds the per 4-row group gate sums and then their
//   exclusive prefix (float [16][DK]), until the Kg rows are written;
// - once A and P are formed, Kn and Qg (tok[1..2]) are dead and hold V
//   (token rows in fragment order, channels in order), the -A strictly-lower
//   blocks, the inverses (I + A_II)^{-1} and T Diag(beta) (upper blocks
//   zero); Kg stays for W = T Kg.
constexpr int kVtOff = 0;                          // V: C token rows x TS (room for d_k rows x CS)
constexpr int kAnOff = kVtOff + DK * CS;           // 6 blocks
constexpr int kDinvOff = kAnOff + 6 * 16 * BS;     // 4 blocks
constexpr int kTbOff = kDinvOff + 4 * 16 * BS;     // 64 rows x CS
static_assert(kTbOff + C * CS <= 2 * C * TS, "V and T fit in two token arrays");
static_assert(C * TS <= DK * CS, "token-major V fits before the -A blocks");
static_assert(kAnOff % 8 == 0 && kDinvOff % 8 == 0 && kTbOff % 8 == 0, "16-byte aligned");
static_assert(16 * DK * sizeof(float) <= C * TS * sizeof(uint16_t), "gate sums fit in one token array");
static_assert(sizeof(PrepSmem) * 3 <= 160 * 1024, "three work-groups per CU");

__device__ __forceinline__ float* gate_sums(PrepSmem& sm) { return reinterpret_cast<float*>(sm.tok[0]); }
__device__ __forceinline__ uint16_t* spare_rows(PrepSmem& sm) { return &sm.tok[0][0] + C * TS; }
__device__ __forceinline__ const uint16_t* spare_rows(const PrepSmem& sm) { return &sm.tok[0][0] + C * TS; }

// 16x16 product of two 16-row blocks stored in fragment order:
// D[m][n] = sum_c X[m][c] Y[n][c]
__device__ __forceinline__ f32x4 row_product(const uint16_t* x, const uint16_t* y, int g, int ln) {
    const uint16_t* xr = x + ln * TS + 8 * g;
    const uint16_t* yr = y + ln * TS + 8 * g;
    u32x4 xf[4], yf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        xf[kk] = *reinterpret_cast<const u32x4*>(xr + 32 * kk);
        yf[kk] = *reinterpret_cast<const u32x4*>(yr + 32 * kk);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mma32(xf[kk], yf[kk], acc);
    return acc;
}

// ---- the exact pairwise form of the decay-weighted products ----
// The factored operands Kg = K e^{g} and Kn = K e^{-g} stay inside fp32
// only while every |g| of the chunk is below kSafeLog2 (log2 units; e^{80}):
// beyond that a channel's e^{-g} overflows, although every factor the
// products need, e^{g_r - g_s} with s <= r, lies in (0, 1].  Such a chunk
// takes this path instead: each entry of A and P is summed over the
// channels with its own factor,
//   Araw[r][s] = sum_c k_r[c] k_s[c] e^{g_r[c] - g_s[c]}        (s <= r)
//   P[r][s]    = sum_c q_r[c] k_s[c] e^{g_r[c] - g_s[c]}
// into fp32 tables that the tile jobs read in place of their matrix-core
// products.  Two forms, by how far the gates go:
// - blocked (every 16-row block's own gate span in range): the factors split
//   at a reference gate rho_I, the cumulative gate just before row block I,
//   e^{g_r - g_s} = e^{g_r - rho_I} e^{rho_I - g_s} for r in block I and
//   s in block J <= I.  For J < I both factors are <= 1; for J = I the
//   second is at most e^{the block's span}, in range by the condition.  So
//   the tiles of row block I are again matrix-core products, of
//   X_I = K_I e^{g - rho_I} (and Q_I e^{g - rho_I}) with
//   Y_J^(I) = K_J e^{rho_I - g}, staged as bf16 32 channels at a time;
// - pairwise (otherwise): each entry summed over the channels with its own
//   factor on the vector units (kda_exact.h).
// Any per-token gate is then in range.
constexpr float kSafeLog2 = 115.f;
constexpr int XS = kExactXS;    // fp32 stride of the staged 32-channel rows
constexpr int AS = C + 1;       // fp32 stride of the 64 x 64 tables

constexpr int BRS = 40;         // bf16 stride of the blocked form's staged rows (32 channels)
static_assert((2 * C + 160) * BRS * sizeof(uint16_t) <= 2 * C * TS * sizeof(uint16_t),
              "the blocked form's staged rows fit in tok[1..2]");

__device__ __forceinline__ float* table_a(PrepSmem& sm) { return reinterpret_cast<float*>(sm.tok[1]); }
__device__ __forceinline__ float* table_p(PrepSmem& sm) { return reinterpret_cast<float*>(sm.tok[1]) + C * AS; }
static_assert(2 * C * AS * sizeof(float) <= 2 * C * TS * sizeof(uint16_t), "the tables fit in tok[1..2]");
static_assert(3 * C * XS * sizeof(float) <= 2 * C * TS * sizeof(uint16_t), "a staged round fits in tok[1..2]");

// Every thread reloads its 4 rows x 4 channels of k and q (normalised by
// nk, nq when the front-end asks) and their gates from L2 once, and rewrites
// its part of Kd^T in the slot with e^{G - g} as one exponential (the common
// path's e^{G} e^{-g} may overflow here).  Then, in 4 rounds of 32 channels,
// BLOCKED: the threads stage X, Q X and the Y^(I) as bf16 rows of BRS, and
// wave w accumulates the A and P tiles w, w + 8, w + 16 (of 20) with one
// matrix-core step per round.  Otherwise they stage k, q and the cumulative
// gates as rows of XS floats for kda_exact.h's pairwise sums.  Called by every thread after a barrier that ends all reads of
// tok[1..2]; returns after the barrier that publishes the tables.  Its
// loops stay rolled: a small register footprint keeps the common path's
// allocation as it is.
template <int GATE, bool FRONT, bool BLOCKED>
__device__ __forceinline__
void exact_ap_tables(PrepSmem& sm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const float* __restrict__ log_alpha, const uint16_t* __restrict__ gate_pre,
                     float gate_scale, int64_t c0, int H, int h, int len, f32x4 off, f32x4 nk,
                     f32x4 nq, uint8_t* __restrict__ out)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int cg = lane & 31;
    const int rg = 2 * (tid >> 6) + (lane >> 5);
    float* sk = reinterpret_cast<float*>(sm.tok[1]);
    float* sq = sk + C * XS;
    float* sg = sq + C * XS;
    // blocked form: bf16 rows of 32 channels (X, Q X, then Y^(I) for I = 0..3,
    // 16 (I + 1) rows each)
    uint16_t* bx = sm.tok[1];
    uint16_t* bqx = bx + C * BRS;
    uint16_t* by = bqx + C * BRS;
    const int wave = tid >> 6, g = lane >> 4, ln = lane & 15;
    f32x4 acc[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    const ExactUnit u = exact_unit(tid);
    float a[4][2], pp[4][2];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) a[x][y] = pp[x][y] = 0.f;
    // this thread's 4 rows x 4 channels, loaded once: k and q as bf16 (each
    // row's 4 channels in one 64-bit word, channel j in bits 16j..) and the
    // cumulative gates in log2 units (off plus the sum within the 4 rows)
    uint64_t kw[4], qw[4];
    f32x4 gl[4];
    {
        const int64_t e0 = (c0 * H + h) * DK;
        const uint32_t span = static_cast<uint32_t>((len - 1) * H * DK + DK);
        f32x4 la[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            if (FRONT && gate_pre) {
                if constexpr (GATE == kGateChannel) {
                    const u32x2 w = ld64(rsrc(gate_pre + e0, 2u * span), 2 * (r * H * DK + 4 * cg));
                    la[i] = f32x4{-gate_scale * softplus_f32(lo_bf(w[0])),
                                  -gate_scale * softplus_f32(hi_bf(w[0])),
                                  -gate_scale * softplus_f32(lo_bf(w[1])),
                                  -gate_scale * softplus_f32(hi_bf(w[1]))};
                } else {
                    const float x = -gate_scale * softplus_f32(bf16_to_f32(ld16(
                        rsrc(gate_pre + c0 * H + h, 2u * static_cast<uint32_t>((len - 1) * H + 1)),
                        2 * r * H)));
                    la[i] = f32x4{x, x, x, x};
                }
                if (r >= len) la[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else if constexpr (GATE == kGateChannel) {
                la[i] = __builtin_bit_cast(f32x4, ld128(rsrc(log_alpha + e0, 4u * span),
                                                        4 * (r * H * DK + 4 * cg)));
            } else {
                const float x = log_alpha
                    ? __uint_as_float(ld32(rsrc(log_alpha + c0 * H + h,
                                                4u * static_cast<uint32_t>((len - 1) * H + 1)),
                                           4 * r * H))
                    : 0.f;
                la[i] = f32x4{x, x, x, x};
            }
            kw[i] = __builtin_bit_cast(uint64_t, ld64(rsrc(k + e0, 2u * span), 2 * (r * H * DK + 4 * cg)));
            qw[i] = __builtin_bit_cast(uint64_t, ld64(rsrc(q + e0, 2u * span), 2 * (r * H * DK + 4 * cg)));
        }
        f32x4 gsum = {0.f, 0.f, 0.f, 0.f};
        float kd[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gsum[j] = __builtin_fmaf(la[i][j], kLog2e, gsum[j]);
                gl[i][j] = off[j] + gsum[j];
                float kx = lo_bf(static_cast<uint32_t>(kw[i] >> (16 * j)));
                if constexpr (FRONT) kx *= nk[i];
                kd[i][j] = kx * __builtin_amdgcn_exp2f(sm.glog[4 * cg + j] - gl[i][j]);
            }
        }
        // Kd^T as the A operand of pass 2 (the common path's layout)
        const int x = 4 * rg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * cg + j;
            const int fl = 16 * ((x & 15) >> 2) + (c & 15);
            *reinterpret_cast<u32x2*>(out + (kFragK + 2 * (c >> 4) + (x >> 5)) * kFrag + fl * 16 +
                                      8 * ((x & 31) >> 4)) =
                u32x2{pk(kd[0][j], kd[1][j]), pk(kd[2][j], kd[3][j])};
        }
    }
    // round j takes channel 4 cg + j of every thread (column cg of the staged
    // rows): any split of the channels into 4 sets of 32 sums to the same
    // tables, and this one keeps every thread busy in every round.  After a
    // round each thread's words and gates move down by one channel.
#pragma unroll 1
    for (int round = 0; round < 4; ++round) {
        if (round > 0) __syncthreads();                 // the last round's reads are done
        const int ch = 4 * cg + round;
        float rho[3];
        if constexpr (BLOCKED) {
#pragma unroll
            for (int I = 0; I < 3; ++I) rho[I] = sm.rho[I][ch];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            float kx = lo_bf(static_cast<uint32_t>(kw[i]));
            float qx = lo_bf(static_cast<uint32_t>(qw[i]));
            if constexpr (FRONT) {
                kx *= nk[i];
                qx *= nq[i];
            }
            const float gr = gl[i][0];
            if constexpr (BLOCKED) {
                const int Ir = rg >> 2;                 // the row block of all 4 rows
                const float f = __builtin_amdgcn_exp2f(gr - (Ir == 0 ? 0.f : rho[Ir - 1]));
                bx[r * BRS + cg] = bf(kx * f);
                bqx[r * BRS + cg] = bf(qx * f);
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if (I < Ir) continue;
                    const float rI = I == 0 ? 0.f : rho[I - 1];
                    by[(8 * I * (I + 1) + r) * BRS + cg] = bf(kx * __builtin_amdgcn_exp2f(rI - gr));
                }
            } else {
                sk[r * XS + cg] = kx;
                sq[r * XS + cg] = qx;
                sg[r * XS + cg] = gr;
            }
            kw[i] >>= 16;
            qw[i] >>= 16;
            gl[i] = f32x4{gl[i][1], gl[i][2], gl[i][3], 0.f};
        }
        __syncthreads();
        if constexpr (BLOCKED) {
            // tiles t = wave, wave + 8, wave + 16 of the 20: A (I, J) for t < 10,
            // P (I, J) for t >= 10, lower tiles numbered row by row
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int t = wave + 8 * x;
                if (t >= 20) continue;
                const int tt = t < 10 ? t : t - 10;
                const int I = (tt >= 1) + (tt >= 3) + (tt >= 6), J = tt - I * (I + 1) / 2;
                const uint16_t* xs = (t < 10 ? bx : bqx) + (16 * I + ln) * BRS + 8 * g;
                const uint16_t* ys = by + (8 * I * (I + 1) + 16 * J + ln) * BRS + 8 * g;
                acc[x] = mma32(*reinterpret_cast<const u32x4*>(xs), *reinterpret_cast<const u32x4*>(ys),
                               acc[x]);
            }
        } else {
            exact_accumulate(u, sk, sq, sg, 1.f, a, pp);
        }
    }
    if constexpr (!BLOCKED) exact_reduce(u, a, pp);
    __syncthreads();                                    // the staged rows are dead
    float* ta = table_a(sm);
    float* tp = table_p(sm);
    if constexpr (BLOCKED) {
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int t = wave + 8 * x;
            if (t >= 20) continue;
            const int tt = t < 10 ? t : t - 10;
            const int I = (tt >= 1) + (tt >= 3) + (tt >= 6), J = tt - I * (I + 1) / 2;
            float* tab = t < 10 ? ta : tp;
#pragma unroll
            for (int i = 0; i < 4; ++i) tab[(16 * I + 4 * g + i) * AS + 16 * J + ln] = acc[x][i];
        }
    } else if (exact_writer(u, tid)) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                ta[(4 * u.bi + x) * AS + 2 * u.bj + y] = a[x][y];
                tp[(4 * u.bi + x) * AS + 2 * u.bj + y] = pp[x][y];
            }
    }
    __syncthreads();
}

// a = (Kg_I Kn_I^T)[4g+i][ln] and at = (Kg_I Kn_I^T)[ln][4g+i] from the
// matrix cores, or from the exact table when the chunk takes that form
template <bool EXACT>
__device__ __forceinline__ u32x2 diag_inverse(const PrepSmem& sm, int I, int g, int ln) {
    f32x4 a, at;
    if constexpr (EXACT) {
        const float* ta = reinterpret_cast<const float*>(sm.tok[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = ta[(16 * I + 4 * g + i) * AS + 16 * I + ln];
            at[i] = ta[(16 * I + ln) * AS + 16 * I + 4 * g + i];
        }
    } else {
        const uint16_t* kgI = sm.tok[0] + 16 * I * TS;
        const uint16_t* knI = sm.tok[1] + 16 * I * TS;
        a = row_product(kgI, knI, g, ln);
        at = row_product(knI, kgI, g, ln);
    }
    const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta + 16 * I + 4 * g);
    const float bl = sm.beta[16 * I + ln];
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
    return pack2(Z3);
}

// the six strictly-lower 16x16 blocks (I > J), numbered I (I - 1) / 2 + J
__device__ __forceinline__ int an_index(int I, int J) { return I * (I - 1) / 2 + J; }

// Column J of T = (I + A)^{-1} below the diagonal by block forward
// substitution, T_IJ = (I + A_II)^{-1} sum_{J<=K<I} (-A_IK) T_KJ, then
// T Diag(beta) into the fragment-ordered rows of tb.
template <int J>
__device__ __forceinline__ void t_column(PrepSmem& sm, int g, int ln) {
    const uint16_t* an = spare_rows(sm) + kAnOff;
    const uint16_t* dinv = spare_rows(sm) + kDinvOff;
    uint16_t* tb = spare_rows(sm) + kTbOff;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 col[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)          // T_JJ = (I + A_JJ)^{-1}, accumulator layout
        col[J][i] = lo_bf(dinv[(16 * J + 4 * g + i) * BS + ln]);
#pragma unroll
    for (int I = J + 1; I < 4; ++I) {
        f32x4 z = zero;
#pragma unroll
        for (int K = J; K < I; ++K)
            z = mma16(*reinterpret_cast<const u32x2*>(an + (an_index(I, K) * 16 + ln) * BS + 4 * g),
                      pack2(col[K]), z);
        col[I] = mma16(*reinterpret_cast<const u32x2*>(dinv + (16 * I + ln) * BS + 4 * g),
                       pack2(z), zero);
    }
    const float bj = sm.beta[16 * J + ln];
    const int cpos = fpos(16 * J + ln);
#pragma unroll
    for (int I = J; I < 4; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i) tb[(16 * I + 4 * g + i) * CS + cpos] = bf(col[I][i] * bj);
    // the upper blocks the products of pass 1 read: (0,1) and (2,3)
    if (J == 1 || J == 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tb[(16 * (J - 1) + 4 * g + i) * CS + cpos] = 0;
    }
}

}  // namespace

// FRONT: the fused input front-end (a separate instantiation, so the plain
// prep is unchanged): q and k L2-normalised per row when fe.l2norm, gates
// from bf16 pre-activations (log_alpha = -fe.gate_scale softplus(x)) when
// fe.gate_pre, beta = sigmoid(y) from bf16 fe.beta_pre
template <int GATE, bool FRONT>
__global__ __launch_bounds__(PT, 4)
void prefill_wy_prep_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                            const bf16_t* __restrict__ v, const float* __restrict__ log_alpha,
                            const float* __restrict__ beta, const int32_t* __restrict__ cu,
                            int H, int DV, int c_lo, int L_b, uint8_t* __restrict__ ws,
                            FrontEnd fe)
{
    __shared__ PrepSmem sm;
    const int slot = blockIdx.x;
    const int h = slot % H;
    const int q_ = slot / H;
    const int n = q_ / L_b;
    const int m = c_lo + q_ % L_b;
    const int64_t t_begin = cu[n];
    const int64_t t_end = cu[n + 1];
    const int64_t c0 = t_begin + static_cast<int64_t>(m) * C;
    if (c0 >= t_end) return;
    const int len = static_cast<int>(min<int64_t>(C, t_end - c0));
    uint8_t* out = ws + static_cast<size_t>(slot) * slot_bytes(DV);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int cg = lane & 31;                  // staging: channels 4cg .. 4cg+3
    const int rg = 2 * wave + (lane >> 5);     //          rows 4rg .. 4rg+3
    if (tid == 0) sm.exact = sm.pairwise = 0;

    // ---------------- staging loads (rows past the end read zero) ----------
    const int64_t e0 = (c0 * H + h) * DK;
    const uint32_t span = static_cast<uint32_t>((len - 1) * H * DK + DK);
    const __amdgpu_buffer_rsrc_t rk = rsrc(k + e0, 2u * span);
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + e0, 2u * span);
    // gates per key channel, or one per (token, head); none (a null
    // log_alpha) gives an empty range, where every load reads zero
    const __amdgpu_buffer_rsrc_t rla =
        GATE == kGateChannel ? rsrc(log_alpha + e0, 4u * span)
        : log_alpha          ? rsrc(log_alpha + c0 * H + h, 4u * static_cast<uint32_t>((len - 1) * H + 1))
                             : rsrc(log_alpha, 0u);
    const __amdgpu_buffer_rsrc_t rv =
        rsrc(v + (c0 * H + h) * DV, 2u * static_cast<uint32_t>((len - 1) * H * DV + DV));
    u32x2 kr[4], qr[4], vr[4];
    f32x4 la[4];
    // the gates first: the cumulative sum waits on them
    if (FRONT && fe.gate_pre) {
        // bf16 pre-activations in the same layout: log_alpha = -c softplus(x)
        const bf16_t* gp = reinterpret_cast<const bf16_t*>(fe.gate_pre);
        const __amdgpu_buffer_rsrc_t rgp =
            GATE == kGateChannel ? rsrc(gp + e0, 2u * span)
                                 : rsrc(gp + c0 * H + h, 2u * static_cast<uint32_t>((len - 1) * H + 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (GATE == kGateChannel) {
                const u32x2 w = ld64_stream(rgp, 2 * ((4 * rg + i) * H * DK + 4 * cg));
                la[i] = f32x4{-fe.gate_scale * softplus_f32(lo_bf(w[0])),
                              -fe.gate_scale * softplus_f32(hi_bf(w[0])),
                              -fe.gate_scale * softplus_f32(lo_bf(w[1])),
                              -fe.gate_scale * softplus_f32(hi_bf(w[1]))};
            } else {
                const float x = -fe.gate_scale *
                                softplus_f32(bf16_to_f32(ld16(rgp, 2 * (4 * rg + i) * H)));
                la[i] = f32x4{x, x, x, x};
            }
            // rows past the end read a zero pre-activation: keep their gate 0
            if (4 * rg + i >= len) la[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (GATE == kGateChannel) {
                la[i] = __builtin_bit_cast(f32x4, ld128_stream(rla, 4 * ((4 * rg + i) * H * DK + 4 * cg)));
            } else {                                  // the row's scalar gate on every channel
                const float x = __uint_as_float(ld32(rla, 4 * (4 * rg + i) * H));
                la[i] = f32x4{x, x, x, x};
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        const int off = r * H * DK + 4 * cg;
        kr[i] = ld64(rk, 2 * off);
        qr[i] = ld64(rq, 2 * off);
        vr[i] = (4 * cg < DV) ? ld64(rv, 2 * (r * H * DV + 4 * cg)) : u32x2{0u, 0u};
    }
    if (tid < C) {
        if (FRONT && fe.beta_pre) {
            const __amdgpu_buffer_rsrc_t rb = rsrc(fe.beta_pre + c0 * H + h,
                                                   2u * static_cast<uint32_t>((len - 1) * H + 1));
            const float y = bf16_to_f32(ld16(rb, 2 * tid * H));
            sm.beta[tid] = tid < len ? sigmoid_f32(y) : 0.f;
        } else {
            const __amdgpu_buffer_rsrc_t rb =
                rsrc(beta + c0 * H + h, 4u * static_cast<uint32_t>((len - 1) * H + 1));
            sm.beta[tid] = __uint_as_float(ld32(rb, 4 * tid * H));
        }
    }
    // L2 norms of the 4 rows' k and q: a row is spread over the 32 lanes of
    // this half-wave, 4 channels each
    float nk[4] = {1.f, 1.f, 1.f, 1.f}, nq[4] = {1.f, 1.f, 1.f, 1.f};
    if (FRONT && fe.l2norm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float kx = (j & 1) ? hi_bf(kr[i][j >> 1]) : lo_bf(kr[i][j >> 1]);
                const float qx = (j & 1) ? hi_bf(qr[i][j >> 1]) : lo_bf(qr[i][j >> 1]);
                sk += kx * kx;
                sq += qx * qx;
            }
#pragma unroll
            for (int m = 1; m < 32; m <<= 1) {
                sk += __shfl_xor(sk, m);
                sq += __shfl_xor(sq, m);
            }
            nk[i] = __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(sk), kFrontEps));
            nq[i] = __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(sq), kFrontEps));
        }
    }

    // ---------------- cumulative gate (log2 units) ----------------------------
    float p[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run = __builtin_fmaf(la[i][j], kLog2e, run);
            p[i][j] = run;
        }
    }
    float* scan = gate_sums(sm);
    *reinterpret_cast<f32x4*>(scan + rg * DK + 4 * cg) = f32x4{p[3][0], p[3][1], p[3][2], p[3][3]};
    __syncthreads();
    if (tid < DK) {
        float run = 0.f, start = 0.f;
        bool far = false;                       // a 16-row block spans beyond the range
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            if (x > 0 && (x & 3) == 0) {
                sm.rho[(x >> 2) - 1][tid] = run;
                far |= !(fabsf(run - start) <= kSafeLog2);
                start = run;
            }
            const float t = scan[x * DK + tid];
            scan[x * DK + tid] = run;
            run += t;
        }
        far |= !(fabsf(run - start) <= kSafeLog2);
        if (far) sm.pairwise = 1;
        sm.glog[tid] = run;
        reinterpret_cast<float*>(out + kOffGam)[tid] = __builtin_amdgcn_exp2f(run);
    }
    __syncthreads();

    // ---------------- decay-weighted operands ---------------------------------
    const f32x4 off = *reinterpret_cast<const f32x4*>(scan + rg * DK + 4 * cg);
    const f32x4 G = *reinterpret_cast<const f32x4*>(&sm.glog[4 * cg]);
    f32x4 gamma;                                // e^{G} of the 4 channels
#pragma unroll
    for (int j = 0; j < 4; ++j) gamma[j] = __builtin_amdgcn_exp2f(G[j]);
    const int cpos = fpos(4 * cg);              // the 4 channels' position in a token row
    // wild: outside the factored form's range anywhere in this thread's
    // part of the chunk (NaN counts as outside)
    bool wild = false;
    float kg[4][4], kd[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        float qg[4], kn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float gl = off[j] + p[i][j];
            const float u = __builtin_amdgcn_exp2f(gl);
            const float w = __builtin_amdgcn_exp2f(-gl);
            // e^{G - g} as e^{G} e^{-g}: both factors stay in range unless the
            // chunk is wild, where the exact form rewrites Kd^T directly
            wild |= !(fabsf(gl) <= kSafeLog2 && fabsf(G[j]) <= kSafeLog2);
            const float d = gamma[j] * w;
            const uint32_t kw = kr[i][j >> 1], qw = qr[i][j >> 1];
            float kx = (j & 1) ? hi_bf(kw) : lo_bf(kw);
            float qx = (j & 1) ? hi_bf(qw) : lo_bf(qw);
            if constexpr (FRONT) {
                kx *= nk[i];
                qx *= nq[i];
            }
            kg[i][j] = kx * u;
            qg[j] = qx * u;
            kn[j] = kx * w;
            kd[i][j] = kx * d;
        }
        *reinterpret_cast<u32x2*>(sm.tok[1] + r * TS + cpos) =
            u32x2{pk(kn[0], kn[1]), pk(kn[2], kn[3])};
        *reinterpret_cast<u32x2*>(sm.tok[2] + r * TS + cpos) =
            u32x2{pk(qg[0], qg[1]), pk(qg[2], qg[3])};
    }
    if (wild) sm.exact = 1;
    {
        const int x = 4 * rg;                   // first of this thread's 4 tokens
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * cg + j;
            // Kd^T as the A operand of pass 2: fragment (m = c/16, kk = x/32),
            // lane (g = (x%16)/4, c%16), half (x%32)/16
            const int fl = 16 * ((x & 15) >> 2) + (c & 15);
            *reinterpret_cast<u32x2*>(out + (kFragK + 2 * (c >> 4) + (x >> 5)) * kFrag + fl * 16 +
                                      8 * ((x & 31) >> 4)) =
                u32x2{pk(kd[0][j], kd[1][j]), pk(kd[2][j], kd[3][j])};
        }
    }
    __syncthreads();   // every gate offset has been read: tok[0] takes the Kg rows
    const bool exact = sm.exact != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x2*>(sm.tok[0] + (4 * rg + i) * TS + cpos) =
            u32x2{pk(kg[i][0], kg[i][1]), pk(kg[i][2], kg[i][3])};
    __syncthreads();

    // Qg as the A operands of pass 2: its token rows are already in fragment
    // order, so fragment (I, kk), lane (g, ln) is 16 contiguous bytes of row
    // 16I + ln; 1024 units, two per thread
#pragma unroll
    for (int x = 0; x < 1024 / PT; ++x) {
        const int u = tid + PT * x;                 // unit = (I, kk, lane)
        const int f = u >> 6, ul = u & 63;
        const int I = f >> 2, kk = f & 3;
        *reinterpret_cast<u32x4*>(out + (kFragQ + f) * kFrag + ul * 16) =
            *reinterpret_cast<const u32x4*>(sm.tok[2] + (16 * I + (ul & 15)) * TS + 32 * kk + 8 * (ul >> 4));
    }

    if (exact) {
        __syncthreads();   // the copy above has read the Qg rows
        const f32x4 nk4{nk[0], nk[1], nk[2], nk[3]}, nq4{nq[0], nq[1], nq[2], nq[3]};
        if (sm.pairwise)
            exact_ap_tables<GATE, FRONT, false>(sm, q, k, log_alpha, fe.gate_pre, fe.gate_scale, c0, H, h,
                                                len, off, nk4, nq4, out);
        else
            exact_ap_tables<GATE, FRONT, true>(sm, q, k, log_alpha, fe.gate_pre, fe.gate_scale, c0, H, h,
                                               len, off, nk4, nq4, out);
    }

    // ---------------- A and P tiles, diagonal inverses ---------------------------
    // jobs 0..5: strictly-lower A blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2);
    // jobs 6..15: lower P blocks (0,0) (1,0) (1,1) (2,0) .. (3,3).  Waves 0..3
    // invert diagonal block I = wave and take job 12 + wave; waves 4..7 take
    // jobs wave-4, wave and wave+4.
    // The exact form reads the tables instead of the matrix cores: a
    // separate instantiation of the jobs, so the common path's code and
    // registers stay as they are.
    u32x2 dres = {0u, 0u};
    f32x4 aval[2];
    int aidx[2] = {-1, -1};
    auto jobs = [&](auto exact_form) {
        constexpr bool EX = decltype(exact_form)::value;
        const float* tab_a = table_a(sm);
        const float* tab_p = table_p(sm);
        if (wave < 4) dres = diag_inverse<EX>(sm, wave, g, ln);
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int j = wave < 4 ? (x == 0 ? 12 + wave : -1) : wave - 4 + 4 * x;
            if (j < 0) continue;
            if (j < 6) {
                const int I = j < 1 ? 1 : j < 3 ? 2 : 3;
                const int J = j - an_index(I, 0);
                f32x4 acc;
                if constexpr (EX) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = tab_a[(16 * I + 4 * g + i) * AS + 16 * J + ln];
                } else {
                    acc = row_product(sm.tok[0] + 16 * I * TS, sm.tok[1] + 16 * J * TS, g, ln);
                }
                const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.beta + 16 * I + 4 * g);
                const int slotx = x == 0 ? 0 : 1;      // jobs j < 6 come at x = 0 and x = 1
                aval[slotx] = -bt * acc;
                aidx[slotx] = j;
            } else {
                const int t = j - 6;
                const int I = (t >= 1) + (t >= 3) + (t >= 6);
                const int J = t - I * (I + 1) / 2;
                // P^T block: acc[i] = P[16I + ln][16J + 4g + i]; diagonal blocks keep s <= r
                f32x4 acc;
                if constexpr (EX) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = tab_p[(16 * I + ln) * AS + 16 * J + 4 * g + i];
                } else {
                    acc = row_product(sm.tok[1] + 16 * J * TS, sm.tok[2] + 16 * I * TS, g, ln);
                }
                u32x2 pv = pack2(acc);
                if (I == J) {
                    f32x4 mk;
#pragma unroll
                    for (int i = 0; i < 4; ++i) mk[i] = (4 * g + i <= ln) ? acc[i] : 0.f;
                    pv = pack2(mk);
                }
                *reinterpret_cast<u32x2*>(out + (kFragP + p_frag(I, J >> 1)) * kFrag + lane * 16 +
                                          8 * (J & 1)) = pv;
            }
        }
    };
    if (exact) jobs(std::true_type{});
    else jobs(std::false_type{});
    if (wave == 0 || wave == 2)   // zero upper halves of the P operands (0,0) and (2,1)
        *reinterpret_cast<u32x2*>(out + (kFragP + p_frag(wave, wave >> 1)) * kFrag + lane * 16 + 8) =
            u32x2{0u, 0u};
    __syncthreads();

    // ---------------- -A blocks, inverses and V into the freed token rows -------
    {
        uint16_t* an = spare_rows(sm) + kAnOff;
        uint16_t* dinv = spare_rows(sm) + kDinvOff;
        if (wave < 4) *reinterpret_cast<u32x2*>(dinv + (16 * wave + ln) * BS + 4 * g) = dres;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            if (aidx[x] < 0) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) an[(aidx[x] * 16 + 4 * g + i) * BS + ln] = bf(aval[x][i]);
        }
        if (4 * cg < DV) {
            // V token-major, token t in row fpos(t): a thread's 4 tokens are 4
            // consecutive rows, each written as one 8-byte piece of 4
            // channels, so the 32 lanes of a row group fill whole rows (the
            // channel-major copy written before put 32 lanes on two bank
            // offsets, a 16-way conflict)
            uint16_t* vt = spare_rows(sm) + kVtOff;
            const int pos = fpos(4 * rg);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x2*>(vt + (pos + i) * TS + 4 * cg) = vr[i];
        }
    }
    __syncthreads();

    // ---------------- T = (I + A)^{-1} Diag(beta), one block column per wave ----
    if (wave == 0) t_column<0>(sm, g, ln);
    else if (wave == 1) t_column<1>(sm, g, ln);
    else if (wave == 2) t_column<2>(sm, g, ln);
    else if (wave == 3) t_column<3>(sm, g, ln);
    __syncthreads();

    // ---------------- -W = -T Kg (as W^T tiles) and U = T V ---------------------
    const uint16_t* tb = spare_rows(sm) + kTbOff;
    {
        // W^T tile (cb, I): lane gets W[16I + ln][16cb + 4g + i]; channel
        // blocks cb = 2kk, 2kk+1 together form W's A operand (I, kk).  Wave
        // w takes kk = w % 4 and the row blocks I = 2 (w / 4), 2 (w / 4) + 1.
        const int kk2 = wave & 3;
        const int Ib = 2 * (wave >> 2);
        // A operand Kg^T (channel 16 cb + ln, tokens in fragment order),
        // gathered from the token rows of Kg: K-step kk, group g takes the
        // tokens 32 kk + 4g + {0..3} and 32 kk + 16 + 4g + {0..3}
        u32x4 kf[2][2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint16_t* col = sm.tok[0] + (32 * kk + 4 * g) * TS + fpos(16 * (2 * kk2 + c) + ln);
                auto two = [&](int x) {
                    return static_cast<uint32_t>(col[x * TS]) | (static_cast<uint32_t>(col[(x + 1) * TS]) << 16);
                };
                kf[c][kk] = u32x4{two(0), two(2), two(16), two(18)};
            }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = Ib + ii;
            f32x4 acc[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > (I >> 1)) continue;
                    const u32x4 tf = *reinterpret_cast<const u32x4*>(tb + (16 * I + ln) * CS + 32 * kk + 8 * g);
                    acc[c] = mma32(kf[c][kk], tf, acc[c]);
                }
            }
            *reinterpret_cast<u32x4*>(out + (kFragW + 4 * I + kk2) * kFrag + lane * 16) =
                cat(pack2(-acc[0]), pack2(-acc[1]));
        }
    }
    const uint16_t* vt = spare_rows(sm) + kVtOff;
    for (int sl = wave; sl < DV / 16; sl += PT / 64) {
        // B operand of K-step kk: rows 32 kk + 8g .. +7 hold the tokens of
        // fragment order (T's order along K), read down channel 16 sl + ln
        // with the LDS transpose read
        u32x4 vf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vf[kk] = frag_tr(vt + 32 * kk * TS + 16 * sl, TS, lane);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk <= (I >> 1); ++kk) {
                const u32x4 tf = *reinterpret_cast<const u32x4*>(tb + (16 * I + ln) * CS + 32 * kk + 8 * g);
                acc = mma32(tf, vf[kk], acc);
            }
            // accumulator layout: lane gets U[16I + 4g + i][16sl + ln]
            *reinterpret_cast<u32x2*>(out + kOffU + sl * kSlabBytes + (I * 64 + lane) * 8) = pack2(acc);
        }
    }
}

// ===================================================================
// pass 2: carry
// ===================================================================
namespace {
constexpr int CW = 8;              // waves
constexpr int CT = CW * 64;
constexpr int kRotDiv = 8;         // copy-order offsets of the value tiles
constexpr int kMaxTwoPassTile = 32;   // columns per tile (register budget of the loaders)
}  // namespace

// SNAP: the call records state snapshots (a separate instantiation, so the
// plain carry's serial loop carries no trace of them)
template <int TV, bool SNAP>
__global__ __launch_bounds__(CT)
void prefill_wy_carry_kernel(const uint8_t* __restrict__ ws, const float* __restrict__ h0,
                             float* __restrict__ hstate, const int32_t* __restrict__ cu,
                             int64_t groups, int R, int H, int DV, int c_lo, int L_b, int c_end,
                             float scale,
                             bf16_t* __restrict__ o, float* __restrict__ snapshots, int snap_tokens,
                             int snap_cap)
{
    constexpr int NSLAB = TV / 16;           // 16-column state slabs in the tile
    constexpr int NC = NSLAB;                // state waves; as many output waves
    constexpr int NL = CW - 2 * NC;          // loader waves
    constexpr int NU = (kOffU - kStageOff + kSlabBytes * NSLAB) / 16;   // staged 16-byte units per chunk
    constexpr int NPL = (NU + NL * 64 - 1) / (NL * 64);     // units per loader lane
    constexpr int NSET = NPL <= 6 ? 6 : 3;   // loader register sets
    static_assert(NSET % 3 == 0, "chunk j is staged in LDS buffer j % 3");
    static_assert(TV >= 16 && TV <= kMaxTwoPassTile, "tile of 16 or 32 columns");
    // three staging buffers: during iteration x the state waves read chunk
    // x and the W of chunk x+1, the loaders fill chunk x+2
    constexpr int NUP = NPL * NL * 64;      // staged units, padded to whole loader rounds
    __shared__ u32x4 buf[3][NUP];
    // handover from a state wave to its output wave: S0 and E of a chunk as
    // B operands, double-buffered by chunk parity
    __shared__ u32x4 xsb[2][NC][4][64];
    __shared__ u32x2 xeb[2][NC][4][64];
    // O of a chunk (bf16, lane (g, ln) of row block I: row 16I + ln, columns
    // 16 slab + 4g .. +3) from the output wave to the state wave, which
    // stores it: a wave whose global loads are in flight then never has a
    // store in flight as well (the compiler can wait on an in-order count of
    // loads alone, not of loads mixed with stores)
    __shared__ u32x2 xob[2][NC][4][64];

    int64_t pair;
    int tile;
    if (!prefill_map_block(blockIdx.x, groups, R, pair, tile)) return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int h = static_cast<int>(pair % H);
    const int n = static_cast<int>(pair / H);
    const int64_t t_begin = cu[n];
    const int64_t t_end = cu[n + 1];
    const int seq_len = static_cast<int>(t_end - t_begin);   // cu_seqlens are int32
    const int nch = (seq_len + C - 1) / C;
    const int count = min(nch, c_lo + L_b) - c_lo;   // chunks of this block
    const int j0 = tile * TV;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV + j0;
    const float* s_in = c_lo == 0 ? h0 : hstate;

    if (count <= 0) {
        // an empty sequence still gets its final state (h0, or zeros)
        if (c_lo == 0 && nch == 0 && wave < NC) {
            const int jc = wave * 16 + ln;
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t e = sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc;
                    hstate[e] = h0 ? h0[e] : 0.f;
                }
        }
        return;
    }
    auto slot_of = [&](int m) {
        return ws + static_cast<size_t>((static_cast<int64_t>(n) * L_b + (m - c_lo)) * H + h) *
                        slot_bytes(DV);
    };

    if (wave >= 2 * NC) {
        // ======================= loader waves =======================
        const int ll = (wave - 2 * NC) * 64 + lane;
        const int ubase = tile * NSLAB * kSlabBytes;   // this tile's U slabs within the slot's U
        // Every load is unconditional (indices clamped to valid data), so the
        // wait before a store to LDS only covers the loads it needs while the
        // later chunks' loads stay in flight.
        // The R tiles of a pair copy the same slot at the same time; each
        // starts at a different offset so they spread over the L2 channels.
        const int rot = (tile * (NU / kRotDiv)) % NU;
        auto unit = [&](int u) { return u + rot < NU ? u + rot : u + rot - NU; };
        auto fetch = [&](u32x4* r, int m) {
            const uint8_t* s = slot_of(min(m, c_lo + count - 1));
#pragma unroll
            for (int x = 0; x < NPL; ++x) {
                const int u = unit(min(ll + x * NL * 64, NU - 1));
                const int byte = kStageOff + 16 * u + (kStageOff + 16 * u >= kOffU ? ubase : 0);
                r[x] = *reinterpret_cast<const u32x4*>(s + byte);
            }
        };
        auto put = [&](const u32x4* r, int b) {
#pragma unroll
            for (int x = 0; x < NPL; ++x) {
                const int u = ll + x * NL * 64;   // padding units land past NU
                buf[b][u < NU ? unit(u) : u] = r[x];
            }
        };
        // NSET register sets: chunk j lives in set j % NSET from its fetch
        // until its store into LDS
        u32x4 r[NSET][NPL];
        const int m0 = c_lo;
#pragma unroll
        for (int k = 0; k < NSET; ++k) fetch(r[k], m0 + k);
        put(r[0], 0);
        fetch(r[0], m0 + NSET);
        put(r[1], 1);
        fetch(r[1], m0 + NSET + 1);
        __syncthreads();
        // iteration x: store chunk x+2 into the buffer freed by chunk x-1 and
        // fetch chunk x+2+NSET into the same set; past the last chunk the
        // stores go to buffers that are never read again.  Whole rounds of
        // NSET iterations run without an early exit, so every path into the
        // loop header has the same loads in flight and the compiler's waits
        // cover only the set being stored.
        // The stores wait ~256 clocks after the barrier: the state waves
        // read this chunk's fragments from LDS first, and 35 KB of stores
        // queued ahead of those reads lengthen the serial step (1.4 % of a
        // 16-column carry call measured; 0 and 512 clocks are slower).
        int x = 0;
        for (; x + NSET <= count; x += NSET) {
#pragma unroll
            for (int k = 0; k < NSET; ++k) {
                __builtin_amdgcn_s_sleep(4);
                put(r[(k + 2) % NSET], (k + 2) % 3);
                fetch(r[(k + 2) % NSET], m0 + x + k + 2 + NSET);
                __syncthreads();
            }
        }
#pragma unroll
        for (int k = 0; k < NSET - 1; ++k) {    // the remaining count - x < NSET iterations
            if (x + k < count) {
                put(r[(k + 2) % NSET], (k + 2) % 3);
                __syncthreads();
            }
        }
        return;
    }

    const int vrow = H * DV;
    // buffer resource over the outputs of chunk m of this tile; rows past
    // the end of the sequence fall outside it and are dropped
    auto out_rsrc = [&](int m) {
        const int64_t c0 = t_begin + static_cast<int64_t>(m) * C;
        const int len = static_cast<int>(min<int64_t>(C, t_end - c0));
        // (a snapshot-recording call may pass no o: every output store is dropped)
        const uint32_t bytes = 2u * static_cast<uint32_t>((len - 1) * vrow + TV);
        return rsrc(o + (c0 * H + h) * DV + j0, SNAP && !o ? 0u : bytes);
    };
    if (wave < NC) {
        // O of chunk m, written by this slab's output wave into xob[b]
        auto store_o = [&](int m, int b) {
            const __amdgpu_buffer_rsrc_t ro = out_rsrc(m);
#pragma unroll
            for (int I = 0; I < 4; ++I)
                st64(ro, 2 * ((16 * I + ln) * vrow + 16 * wave + 4 * g), xob[b][wave][I][lane]);
        };
        // ======================= state waves =======================
        // fp32 state slab in the accumulator layout:
        // S[m][i] = state[c = 16m + 4g + i][j = j0 + wave * 16 + ln]
        const int jc = wave * 16 + ln;
        f32x4 S[8];
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[m][i] = s_in ? s_in[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc] : 0.f;
        __syncthreads();
        // W of chunk x is read during iteration x-1 (chunk x is staged by
        // then); the other fragments one stage ahead within the iteration
        // (scheduling barriers keep the order); independent accumulators
        // interleave
        u32x4 wf[16];
#pragma unroll
        for (int f = 0; f < 16; ++f) wf[f] = buf[0][f * 64 + lane];
        int bx = 0;                              // x % 3
        // chunks until the next snapshot boundary (snap_tokens is a multiple of C)
        const int snap_stride = SNAP ? snap_tokens / C : 0;
        int snap_left = SNAP ? snap_stride - c_lo % snap_stride : 0;
        for (int x = 0; x < count; ++x) {
            const u32x4* F = buf[bx];
            const int bn = bx == 2 ? 0 : bx + 1;
            const u32x2* U = reinterpret_cast<const u32x2*>(F + (kOffU - kStageOff) / 16) + wave * 4 * 64;
            const float* gam = reinterpret_cast<const float*>(F + (kOffGam - kStageOff) / 16);
            u32x2 uw[4];
            f32x4 gm[8];
#pragma unroll
            for (int I = 0; I < 4; ++I) uw[I] = U[I * 64 + lane];
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) gm[mm] = *reinterpret_cast<const f32x4*>(gam + 16 * mm + 4 * g);
            // Kd^T of this chunk: read ahead of the E products, so it is
            // serviced while they run, before the loaders' stores reach LDS
            // (0.7 % of a call measured)
            u32x4 kf[16];
#pragma unroll
            for (int f = 0; f < 16; ++f) kf[f] = F[(kFragK - kFragW + f) * 64 + lane];
            u32x4 sb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sb[kk] = pack4(S[2 * kk], S[2 * kk + 1]);
            // E = U + (-W) S0, accumulated from U: the MFMAs leave E itself
            f32x4 y[4];
#pragma unroll
            for (int I = 0; I < 4; ++I)
                y[I] = f32x4{lo_bf(uw[I][0]), hi_bf(uw[I][0]), lo_bf(uw[I][1]), hi_bf(uw[I][1])};
            __builtin_amdgcn_sched_barrier(0);

            // ---- E (4 independent chains), with Diag(e^{G}) S0 formed meanwhile
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int I = 0; I < 4; ++I) y[I] = mma32(wf[4 * I + kk], sb[kk], y[I]);
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) S[mm] = gm[mm] * S[mm];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int f = 0; f < 16; ++f) wf[f] = buf[bn][f * 64 + lane];   // -W of chunk x+1
            u32x2 eb[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) eb[I] = pack2(y[I]);
            const u32x4 e01 = cat(eb[0], eb[1]), e23 = cat(eb[2], eb[3]);
            // hand S0 and E of this chunk to the output wave
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) xsb[x & 1][wave][kk][lane] = sb[kk];
#pragma unroll
            for (int I = 0; I < 4; ++I) xeb[x & 1][wave][I][lane] = eb[I];
            __builtin_amdgcn_sched_barrier(0);

            // ---- S = Diag(e^{G}) S0 + Kd^T E
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) S[mm] = mma32(kf[2 * mm], e01, S[mm]);
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) S[mm] = mma32(kf[2 * mm + 1], e23, S[mm]);
            if (x >= 2) store_o(c_lo + x - 2, x & 1);
            // a snapshot after every snap_stride chunks: a countdown, so the
            // serial loop pays one decrement per chunk (buffer stores keep
            // the addressing in scalar registers and one lane offset)
            const int js = SNAP && --snap_left == 0
                               ? (snap_left = snap_stride, (c_lo + x + 1) / snap_stride - 1) : -1;
            // (only a full chunk ends on a boundary).  snap_cap < 0 selects the
            // compact per-chunk record of the gradient pass: bf16 transposed states, the
            // state after chunk js of sequence n at index n + cu[n] / C + js,
            // which never collides with the next sequence's (it starts at
            // least ceil(len / C) indices on)
            if (js >= 0 && (snap_cap < 0 || js < snap_cap) && (c_lo + x + 1) * C <= seq_len) {
                const int64_t SE = static_cast<int64_t>(DK) * DV;
                if (snap_cap >= 0) {
                    // the lane's first element offset, opaque: formed here,
                    // not ahead of the branch on every chunk (32 offsets,
                    // ~70 instructions on the serial path of the record
                    // mode, which never takes this branch)
                    int lo = 4 * g * DV + jc;
                    asm volatile("" : "+v"(lo));
                    float* sp = snapshot_at(snapshots, snap_cap, H, SE, n, js, h);
                    const __amdgpu_buffer_rsrc_t rs = rsrc(sp + j0, 4u * DK * DV);
#pragma unroll
                    for (int m = 0; m < 8; ++m)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            st32(rs, 4 * (lo + (16 * m + i) * DV), __float_as_uint(S[m][i]));
                } else {
                    // bf16, transposed ([value column][key row]): a lane's 4
                    // rows of one column are one 8-byte store
                    bf16_t* sp = reinterpret_cast<bf16_t*>(snapshots) + ((n + t_begin / C + js) * H + h) * SE;
                    const __amdgpu_buffer_rsrc_t rs = rsrc(sp + static_cast<int64_t>(j0) * DK, 2u * TV * DK);
#pragma unroll
                    for (int m = 0; m < 8; ++m) st64(rs, 2 * (jc * DK + 16 * m + 4 * g), pack2(S[m]));
                }
            }
            __syncthreads();
            bx = bn;
        }
        if (count >= 2) store_o(c_lo + count - 2, count & 1);
        // a sequence longer than the call's chunk bound (the caller's
        // max_seqlen) was cut short: its final state is NaN, not a silently
        // wrong state
        const bool cut = c_lo + L_b >= c_end && nch > c_lo + count;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hstate[sbase + static_cast<int64_t>(16 * m + 4 * g + i) * DV + jc] =
                    cut ? __builtin_nanf("") : S[m][i];
        return;
    }

    // ======================= output waves =======================
    // O of chunk x-1 = scale (Qg S0 + P E), during iteration x: from the Qg
    // and P fragments copied in iteration x-1 and the state wave's handover;
    // rows past the end of the sequence are dropped by the range check
    const int sl = wave - NC;                   // slab
    auto out_chunk = [&](int m, const u32x4* qf, const u32x4* pf, int b, bool direct) {
        u32x4 sb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sb[kk] = xsb[b][sl][kk][lane];
        const u32x4 e01 = cat(xeb[b][sl][0][lane], xeb[b][sl][1][lane]);
        const u32x4 e23 = cat(xeb[b][sl][2][lane], xeb[b][sl][3][lane]);
        // O^T = S0^T Qg^T + E^T P^T: the same fragments with the operands
        // swapped (an A-operand lane layout is the transpose of a B-operand
        // one), so lane (g, ln) gets O[16I + ln][16 sl + 4g + i] and stores
        // four adjacent columns of one token row at once
        f32x4 oc[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) oc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int I = 0; I < 4; ++I) oc[I] = mma32(sb[kk], qf[4 * I + kk], oc[I]);
#pragma unroll
        for (int I = 0; I < 4; ++I) oc[I] = mma32(e01, pf[p_frag(I, 0)], oc[I]);
        oc[2] = mma32(e23, pf[p_frag(2, 1)], oc[2]);
        oc[3] = mma32(e23, pf[p_frag(3, 1)], oc[3]);
        if (direct) {
            const __amdgpu_buffer_rsrc_t ro = out_rsrc(m);
#pragma unroll
            for (int I = 0; I < 4; ++I)
                st64(ro, 2 * ((16 * I + ln) * vrow + 16 * sl + 4 * g), pack2(scale * oc[I]));
        } else {
#pragma unroll
            for (int I = 0; I < 4; ++I) xob[b][sl][I][lane] = pack2(scale * oc[I]);
        }
    };
    // Qg and P come from the slot straight into registers, two iterations
    // before they are used: set a holds the block's even chunks, set b the
    // odd ones (loads past the last chunk re-read it and are never used)
    auto load_qp = [&](u32x4* qf, u32x4* pf, int m) {
        const uint8_t* s = slot_of(min(m, c_lo + count - 1)) + lane * 16;
#pragma unroll
        for (int f = 0; f < 16; ++f) qf[f] = *reinterpret_cast<const u32x4*>(s + (kFragQ + f) * kFrag);
#pragma unroll
        for (int f = 0; f < 6; ++f) pf[f] = *reinterpret_cast<const u32x4*>(s + (kFragP + f) * kFrag);
    };
    u32x4 qa[16], pa[6], qb[16], pb[6];
    load_qp(qa, pa, c_lo);
    load_qp(qb, pb, c_lo + 1);
    __syncthreads();
    __syncthreads();                            // iteration 0 has no output
    // iteration x >= 1: O of chunk x-1, whose handover the state wave wrote
    // in iteration x-1, then the loads of chunk x+1 into the set just used.
    // Two iterations per trip and no early exit: every path into the loop
    // header has the same loads in flight, so the compiler's waits cover
    // only the set being consumed.
    int x = 1;
    for (; x + 1 < count; x += 2) {
        out_chunk(c_lo + x - 1, qa, pa, 0, false);
        load_qp(qa, pa, c_lo + x + 1);
        __syncthreads();
        out_chunk(c_lo + x, qb, pb, 1, false);
        load_qp(qb, pb, c_lo + x + 2);
        __syncthreads();
    }
    if (x < count) {                            // iteration count-1 (even chunk count-2)
        out_chunk(c_lo + x - 1, qa, pa, 0, false);
        __syncthreads();
    }
    // the last chunk: its handover was written before the final barrier;
    // its O is stored here (the state wave stores the one before it)
    if ((count - 1) & 1) out_chunk(c_lo + count - 1, qb, pb, 1, true);
    else out_chunk(c_lo + count - 1, qa, pa, 0, true);
}

// ===================================================================
// host side
// ===================================================================
namespace {
// default bytes of slots per block: small enough that a block's slots stay
// resident in the 256 MiB last-level cache between the two passes
constexpr size_t kSlotBudget = size_t{150} << 20;
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t chunk_bound(int64_t total_T) { return total_T > 0 ? (total_T + C - 1) / C : 1; }

template <int TV>
hipError_t launch_carry_t(const PrefillArgs& a, int R, int c_lo, int L_b, int c_end,
                          const uint8_t* slots, float* hstate, hipStream_t stream) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    const int64_t blocks = prefill_grid_blocks(groups, R);
    auto carry = a.snapshots ? prefill_wy_carry_kernel<TV, true> : prefill_wy_carry_kernel<TV, false>;
    hipLaunchKernelGGL(carry, dim3(static_cast<unsigned>(blocks)), dim3(CT),
                       0, stream, slots, a.h0, hstate, a.cu_seqlens, groups, R, a.H, a.d_v, c_lo,
                       L_b, c_end, a.scale, static_cast<bf16_t*>(a.o), a.snapshots, a.snap_tokens, a.snap_cap);
    return hipGetLastError();
}
}  // namespace

bool wy_supported(const PrefillArgs& a) {
    return !a.dtype_f32 && a.d_k == DK && a.H <= kMaxHeads;
}

// Value tiles per (sequence, head): 16 or 32 columns, and enough
// work-groups to cover the 256 compute units where the batch allows.
int wy_value_tiles(const PrefillArgs& a) {
    const int64_t groups = static_cast<int64_t>(a.N) * a.H;
    int R = a.d_v > kMaxTwoPassTile ? a.d_v / kMaxTwoPassTile : 1;
    while (R < a.d_v / 16 && groups * R < 256) R *= 2;
    return R;
}

bool wy_tiles_ok(int d_v, int R) {
    return R > 0 && (R & (R - 1)) == 0 && d_v % R == 0 && d_v / R >= 16 &&
           d_v / R <= kMaxTwoPassTile;
}

int wy_default_block_chunks(int64_t seq_bound, int32_t N, int32_t H, int32_t d_v) {
    const size_t per_chunk = static_cast<size_t>(N) * H * slot_bytes(d_v);
    int64_t L = static_cast<int64_t>(kSlotBudget / per_chunk);
    if (L >= 16) L -= L % 16;
    L = std::max<int64_t>(1, std::min<int64_t>(L, chunk_bound(seq_bound)));
    return static_cast<int>(L);
}

bool wy_block_chunks_ok(int32_t N, int32_t H, int L_b) {
    if (L_b < 1) return false;
    const int64_t slots = static_cast<int64_t>(N) * H * L_b;
    return slots < (int64_t{1} << 31) && slots <= (int64_t{1} << 40) / slot_bytes(128);
}

size_t wy_workspace_bytes(int32_t N, int32_t H, int32_t d_k, int32_t d_v, int L_b) {
    const size_t slots = static_cast<size_t>(N) * H * L_b * slot_bytes(d_v);
    const size_t state = static_cast<size_t>(N) * H * d_k * d_v * sizeof(float);
    return align_up(slots) + align_up(state);
}

hipError_t launch_prefill_wy(const PrefillArgs& a, int R, int L_b, void* ws, hipStream_t stream) {
    uint8_t* slots = static_cast<uint8_t*>(ws);
    const size_t slot_total = align_up(static_cast<size_t>(a.N) * a.H * L_b * slot_bytes(a.d_v));
    float* hstate = a.hT ? a.hT : reinterpret_cast<float*>(slots + slot_total);
    // blocks cover the longest sequence's chunks (the caller's max_seqlen),
    // else every chunk index a sequence of total_T tokens could have
    const int64_t bound = chunk_bound(a.seq_bound());
    const int TV = a.d_v / R;
    for (int64_t c_lo = 0; c_lo < bound; c_lo += L_b) {
        if (a.total_T > 0) {
            const int64_t nslots = static_cast<int64_t>(a.N) * L_b * a.H;
            const bool ch = a.gate == kGateChannel, fr = a.fe.active();
            auto prep = ch ? (fr ? prefill_wy_prep_kernel<kGateChannel, true>
                                 : prefill_wy_prep_kernel<kGateChannel, false>)
                           : (fr ? prefill_wy_prep_kernel<kGateHead, true>
                                 : prefill_wy_prep_kernel<kGateHead, false>);
            hipLaunchKernelGGL(prep, dim3(static_cast<unsigned>(nslots)), dim3(PT),
                               0, stream, static_cast<const bf16_t*>(a.q),
                               static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.v),
                               a.log_alpha, a.beta, a.cu_seqlens, a.H, a.d_v,
                               static_cast<int>(c_lo), L_b, slots, a.fe);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipError_t e = hipErrorInvalidValue;
        switch (TV) {
            case 16: e = launch_carry_t<16>(a, R, static_cast<int>(c_lo), L_b,
                                            static_cast<int>(bound), slots, hstate, stream); break;
            case 32: e = launch_carry_t<32>(a, R, static_cast<int>(c_lo), L_b,
                                            static_cast<int>(bound), slots, hstate, stream); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
