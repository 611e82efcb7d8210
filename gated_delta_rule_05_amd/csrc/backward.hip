// backward.hip -- gradients of the chunked KDA prefill on gfx950.
//
// L = <o, dO> + <hT, dhT>; the gradients of L with respect to q, k, v,
// log_alpha, beta and h0, for the recurrence of "Kimi Delta Attention: la
// atencion lineal detras de Kimi K2 y Qwen3", section "Cómo funciona Kimi
// Delta Attention paso a paso", in its chunked (UT/WY) form.  That page
// names chunkwise computation as the production form of the forward pass;
// "Kimi Linear acaba de superar a la atención completa en sus propios
// términos" (section "Cómo Kimi Linear utiliza una memoria recurrente más
// inteligente") presents the chunkwise algorithm as what makes training
// efficient.  The derivation below is ours.
//
// One chunk (C = 64 rows r, s), S its start state, g the within-chunk
// cumulative log gate, G = g of its last row, Kg = K e^g, Kn = K e^-g,
// Qg = Q e^g, Kd = K e^{G-g}, gamma = e^G:
//     B = Kg Kn^T, A = strict_lower(Diag(beta) B), Minv = (I + A)^-1,
//     T = Minv Diag(beta), R = V - Kg S, E = T R  (= U - W S, U = T V, W = T Kg),
//     P = lower(Qg Kn^T) (diagonal included),
//     O = scale (Qg S + P E),   S' = Diag(gamma) S + Kd^T E.
// Given dO and dS' (the adjoint of the chunk's end state), by reverse-mode
// differentiation of those lines:
//     dE  = Kd dS' + scale P^T dO                            (carry)
//     dS  = Diag(gamma) dS' + scale Qg^T dO - W^T dE         (carry, serial)
//     dV  = T^T dE,  dT = dE R^T,  dKg_W = -dV S^T,  dQg_S = scale dO S^T,
//     dKd = E dS'^T,  dP = lower(scale dO E^T),  dgamma = rowsum(dS' . S),
//     dbeta_T = diag(Minv^T dT),  dA = -strict_lower(Minv^T dT Diag(beta) Minv^T),
//     dB = Diag(beta) dA,  dbeta_A = rowsum(dA . B),
//     dKg = dKg_W + dB Kn,  dKn = dP^T Qg + dB^T Kg,  dQg = dQg_S + dP Kn,
//     dK = dKg e^g + dKn e^-g + dKd e^{G-g},  dQ = dQg e^g,
//     dg = dKg.Kg - dKn.Kn + dQg.Qg - dKd.Kd,  dG = colsum(dKd.Kd) + dgamma.gamma,
//     dlog_alpha[s] = sum_{r >= s} dg[r] + dG,   dbeta = dbeta_T + dbeta_A.
//
// Passes (one call): the forward two-pass prefill records the start state of
// every chunk (no outputs); then, over blocks of chunks from the last:
//   prep   (chunk-parallel) recomputes a chunk's operands: Kd, Kg, scale P^T,
//          scale Qg, -W^T, Minv, gamma;
//   carry  (serial per (sequence, head, 64 value columns)) walks the chunks
//          backwards with dS in registers, storing dS' and dE of each chunk;
//   grad   (chunk-parallel) first the products with the states (dV, dT,
//          dKg_W, dQg_S, dKd, dP, dgamma), kept in registers, then the
//          triangular-system and gate terms and the gradients of q, k,
//          log_alpha and beta.
// Every product is a bf16 MFMA (16x16x32) with fp32 accumulation on
// operands staged in LDS; states, adjoints and gates stay fp32.
#include <algorithm>

#include "kda_device.h"
#include "kda_exact.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int C = 64;          // chunk rows
constexpr int D = 128;         // d_k = d_v
constexpr int NT = 256;        // default work-group size of the LDS helpers
constexpr int GT = 512;        // threads of the prep and the carry: 8 waves, 2 per SIMD
constexpr int GG = 1024;       // threads of the gradient kernel: 16 waves, 4 per SIMD
constexpr int LDD = D + 8;     // padded LDS row of a [.][D] bf16 matrix
constexpr int LDC = C + 8;     // padded LDS row of a [.][C] bf16 matrix
constexpr int kCarryTile = 64; // value columns per carry work-group
constexpr int LDO = kCarryTile + 16;   // the carry's dO tile: rows read by transpose reads

// per-(chunk, head) operands written by the prep pass (bytes)
constexpr int kOffKd = 0;                    // [C][D] bf16   K e^{G-g}
constexpr int kOffKg = kOffKd + C * D * 2;   // [C][D] bf16   K e^{g}
constexpr int kOffPt = kOffKg + C * D * 2;   // [C][C] bf16   scale P^T
constexpr int kOffQg = kOffPt + C * C * 2;   // [C][D] bf16   scale Qg
constexpr int kOffWt = kOffQg + C * D * 2;   // [D][C] bf16   -W^T
constexpr int kOffMinv = kOffWt + D * C * 2; // [C][C] fp32   (I + A)^-1
constexpr int kOffGam = kOffMinv + C * C * 4; // [D]    fp32   e^{G}
constexpr int kSlot = kOffGam + D * 4;
constexpr int64_t kState = static_cast<int64_t>(D) * D;   // floats per state

static_assert(kSlot % 256 == 0, "256-byte aligned records");

// ---- the chunk a work-group of a chunk-parallel pass owns
struct ChunkRef {
    int n, h, j, len;     // sequence, head, chunk index in the sequence, rows
    int64_t t0;           // first token
    int64_t slot;         // (sequence, chunk in block, head) record index
};
__device__ __forceinline__ bool chunk_of(int64_t b, int H, int c_lo, int L_b,
                                         const int32_t* cu, ChunkRef& c) {
    c.h = static_cast<int>(b % H);
    const int64_t q = b / H;
    const int jj = static_cast<int>(q % L_b);
    c.n = static_cast<int>(q / L_b);
    c.j = c_lo + jj;
    c.slot = b;
    c.t0 = static_cast<int64_t>(cu[c.n]) + static_cast<int64_t>(c.j) * C;
    const int64_t end = cu[c.n + 1];
    c.len = static_cast<int>(min<int64_t>(C, end - c.t0));
    return c.len > 0;
}

// Operand storage in LDS.  kKc: one row per M (or N) index with K
// contiguous -- lane (g, ln) reads row ln, K indices 8g .. 8g+7 (one 16-byte
// read).  kMc: one row per K index with M (or N) contiguous -- the same
// fragment by two transpose reads (frag_tr).
constexpr int kKc = 0, kMc = 1;

// tile i (16 rows or columns) of an operand stored with layout L
template <int L>
__device__ __forceinline__ const bf16_t* tile_at(const bf16_t* x, int ld, int i) {
    return L == kKc ? x + 16 * i * ld : x + 16 * i;
}
template <int L>
__device__ __forceinline__ u32x4 frag(const bf16_t* x, int ld, int kk, int lane) {
    if constexpr (L == kKc)
        return *reinterpret_cast<const u32x4*>(x + (lane & 15) * ld + 8 * (lane >> 4) + kk);
    else
        return frag_tr(x + kk * ld, ld, lane);
}

// acc(16x16 tile) of A (M x K) times B (K x N), a and b pointing at the
// tile (tile_at), A stored with layout AL and B with layout BL; the kKc
// form of B is B^T (N x K, row n at b + n * ldb).
template <int K, int AL = kKc, int BL = kKc>
__device__ __forceinline__ f32x4 tile_mm(const bf16_t* a, int lda, const bf16_t* b, int ldb,
                                         int lane, f32x4 acc) {
#pragma unroll
    for (int kk = 0; kk < K; kk += 32)
        acc = mma32(frag<AL>(a, lda, kk, lane), frag<BL>(b, ldb, kk, lane), acc);
    return acc;
}

// this wave's tiles of a (MT x NTL)-tile product, in a fixed order: tile x
// is t = wave + W x for W waves (row block t / NTL, column block t % NTL).
// W is a multiple of NTL, so all of a wave's tiles share one column block:
// each B fragment is read from LDS once per K step and used for every tile.
template <int NTL, int K, int NX, int NTH = NT, int AL = kKc, int BL = kKc>
__device__ __forceinline__ void mm_regs(const bf16_t* a, int lda, const bf16_t* b, int ldb,
                                        f32x4 (&out)[NX]) {
    constexpr int W = NTH / 64;
    static_assert(W % NTL == 0, "a wave's tiles in one column block");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m0 = wave / NTL;
    const bf16_t* bt = tile_at<BL>(b, ldb, wave % NTL);
#pragma unroll
    for (int x = 0; x < NX; ++x) out[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < K; kk += 32) {
        const u32x4 fb = frag<BL>(bt, ldb, kk, lane);
#pragma unroll
        for (int x = 0; x < NX; ++x)
            out[x] = mma32(frag<AL>(tile_at<AL>(a, lda, m0 + (W / NTL) * x), lda, kk, lane), fb,
                           out[x]);
    }
}

// all 16x16 tiles (mi < MT, ni < NTL) of A B, spread over the NTH / 64 waves
// as in mm_regs; fn(mi, ni, acc) consumes each (acc[i] = row 16 mi + 4g + i,
// column 16 ni + ln)
template <int MT, int NTL, int K, int NTH = NT, int AL = kKc, int BL = kKc, typename Fn>
__device__ __forceinline__ void mm(const bf16_t* a, int lda, const bf16_t* b, int ldb,
                                   Fn&& fn) {
    constexpr int W = NTH / 64, NX = MT * NTL / W;
    static_assert(MT * NTL % W == 0, "whole tiles per wave");
    f32x4 acc[NX];
    mm_regs<NTL, K, NX, NTH, AL, BL>(a, lda, b, ldb, acc);
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int t = wave + W * x;
        fn(t / NTL, t % NTL, acc[x]);
    }
}

// component j (a constant after unrolling) of a float4
__device__ __forceinline__ float f4_at(const float4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// store 4 values of one column, rows r0..r0+3, into a transposed bf16
// matrix (row = column index): one 8-byte LDS or global store
__device__ __forceinline__ void put4t(bf16_t* p, f32x4 x) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pk(x[0], x[1]), pk(x[2], x[3])};
}


// the raw gates of the thread's 4 x 4 block (zero past the chunk), and
// beta of row tid (tid < C; 0 past the chunk)
template <int GATE>
__device__ __forceinline__ void load_gate_block(const float* la, const float* beta,
                                                const ChunkRef& c, int H, f32x4 (&raw)[4],
                                                float& b) {
    const int tid = threadIdx.x, rg = tid >> 5, cg = tid & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        raw[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (r < c.len) {
            const int64_t row = (c.t0 + r) * H + c.h;
            if constexpr (GATE == kGateChannel) {
                raw[i] = *reinterpret_cast<const f32x4*>(la + row * D + 4 * cg);
            } else if constexpr (GATE == kGateHead) {
                const float a = la[row];
                raw[i] = f32x4{a, a, a, a};
            }
        }
    }
    b = tid < C && tid < c.len ? beta[(c.t0 + tid) * H + c.h] : 0.f;
}

// the scan of chunk_gates over a thread's raw 4 x 4 block (two barriers)
__device__ __forceinline__ void scan_gate_block(const f32x4 (&raw)[4], float b, float* scan,
                                                float* tot, float* bs, float (&g)[4][4],
                                                f32x4& G) {
    static_assert(GT == (C / 4) * (D / 4), "one thread per 4 x 4 block of the chunk");
    const int tid = threadIdx.x, rg = tid >> 5, cg = tid & 31;
    const bool own = tid < GT;    // a larger work-group's other threads only pass the barriers
    if (tid < C) bs[tid] = b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run += raw[i][j];
            g[i][j] = run;
        }
    }
    if (own) *reinterpret_cast<f32x4*>(scan + rg * D + 4 * cg) = f32x4{g[3][0], g[3][1], g[3][2], g[3][3]};
    __syncthreads();
    if (tid < D) {
        float run = 0.f;
#pragma unroll
        for (int x = 0; x < C / 4; ++x) {
            const float t = scan[x * D + tid];
            scan[x * D + tid] = run;
            run += t;
        }
        tot[tid] = run;
    }
    __syncthreads();
    const f32x4 off = own ? *reinterpret_cast<const f32x4*>(scan + rg * D + 4 * cg)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    G = *reinterpret_cast<const f32x4*>(tot + 4 * cg);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) g[i][j] += off[j];
}

// Cumulative gates of a chunk at the thread's 4 rows 4 rg + i and 4
// channels 4 cg + j (rg = tid / 32, cg = tid % 32, all GT threads): each
// thread sums down its own rows, then a scan over the 16 row groups adds the
// groups before.  Rows past the chunk add zero, so they repeat the last row,
// and G (the chunk's total per channel) equals the last row's value.  Beta
// of the rows into bs (0 past the chunk).  scan: 16 x D floats, tot: D
// floats, both LDS; two barriers inside.
template <int GATE>
__device__ __forceinline__ void chunk_gates(const float* la, const float* beta, const ChunkRef& c,
                                            int H, float* scan, float* tot, float* bs,
                                            float (&g)[4][4], f32x4& G) {
    f32x4 raw[4];
    float b;
    load_gate_block<GATE>(la, beta, c, H, raw, b);
    scan_gate_block(raw, b, scan, tot, bs, g, G);
}

// k or q of the thread's 4 rows 4 rg + i, channels 4 cg .. +3 (zero past
// the chunk), as fp32
template <typename T>
__device__ __forceinline__ void load_rows4(const T* x, const ChunkRef& c, int H, float4 (&out)[4]) {
    const int tid = threadIdx.x, rg = tid >> 5, cg = tid & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        out[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < c.len) out[i] = elem<T>::load4(x + ((c.t0 + r) * H + c.h) * D + 4 * cg);
    }
}

// the same block as raw bf16 pairs (half the registers of load_rows4)
__device__ __forceinline__ void load_rows4_raw(const bf16_t* x, const ChunkRef& c, int H,
                                               u32x2 (&out)[4]) {
    const int tid = threadIdx.x, rg = tid >> 5, cg = tid & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        out[i] = u32x2{0u, 0u};
        if (r < c.len) out[i] = *reinterpret_cast<const u32x2*>(x + ((c.t0 + r) * H + c.h) * D + 4 * cg);
    }
}

// ===================================================================
// prep: a chunk's operands for the backward passes
// ===================================================================
// 69 KB, so two work-groups share a CU: buffers whose lives do not overlap
// share LDS (the gate scan, then B; K e^-g and Q e^g, then the inverse)
struct alignas(16) PrepLds {
    bf16_t kg[C * LDD];
    union {
        struct { bf16_t kn[C * LDD], qg[C * LDD]; } a;
        struct {
            float mi[C * (C + 1)];
            bf16_t tt[C * LDC];
            float xs[3][16 * 17];      // one wave's product block of the inverse
        } b;
    } u1;
    union {
        struct { float scan[(C / 4) * D], tot[D]; } a;
        float bm[C * (C + 1)];
    } u2;
    float bs[C];
    int wild;                  // beyond the factored range ...
    int pairwise;              // ... and a 16-row block's own gate sum beyond it too
};

// |g| (natural log units) up to which e^{g} and e^{-g} stay inside fp32
constexpr float kSafeGate = 80.f;
constexpr int BRS = 40;        // bf16 stride of the blocked form's staged rows (32 channels)

template <int GATE>
__global__ __launch_bounds__(GT, 2)
void bwd_prep_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const float* __restrict__ la, const float* __restrict__ beta,
                     const int32_t* __restrict__ cu, int H, int c_lo, int L_b, float scale,
                     uint8_t* __restrict__ slots)
{
    __shared__ PrepLds sm;
    ChunkRef c;
    if (!chunk_of(blockIdx.x, H, c_lo, L_b, cu, c)) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, ln = lane & 15;
    uint8_t* out = slots + c.slot * static_cast<int64_t>(kSlot);
    bf16_t* oKd = reinterpret_cast<bf16_t*>(out + kOffKd);
    bf16_t* oKg = reinterpret_cast<bf16_t*>(out + kOffKg);
    bf16_t* oPt = reinterpret_cast<bf16_t*>(out + kOffPt);
    bf16_t* oQg = reinterpret_cast<bf16_t*>(out + kOffQg);
    bf16_t* oWt = reinterpret_cast<bf16_t*>(out + kOffWt);
    float* oMinv = reinterpret_cast<float*>(out + kOffMinv);
    float* oGam = reinterpret_cast<float*>(out + kOffGam);

    // k and q of the thread's rows load while the gates scan
    const int rg = tid >> 5, cg = tid & 31;
    float4 kr4[4], qr4[4];
    load_rows4(k, c, H, kr4);
    load_rows4(q, c, H, qr4);
    float g[4][4];
    f32x4 G;
    if (tid == 0) sm.wild = sm.pairwise = 0;
    chunk_gates<GATE>(la, beta, c, H, sm.u2.a.scan, sm.u2.a.tot, sm.bs, g, G);
    if (tid < D) {
        oGam[tid] = gate_exp(sm.u2.a.tot[tid]);
        // the gate sums of the four 16-row blocks on channel tid
        const float r1 = sm.u2.a.scan[4 * D + tid], r2 = sm.u2.a.scan[8 * D + tid];
        const float r3 = sm.u2.a.scan[12 * D + tid], gt = sm.u2.a.tot[tid];
        const bool far = !(fabsf(r1) <= kSafeGate && fabsf(r2 - r1) <= kSafeGate &&
                           fabsf(r3 - r2) <= kSafeGate && fabsf(gt - r3) <= kSafeGate);
        if (far) sm.pairwise = 1;
    }
    {
        // the factored form's range: a chunk beyond it takes the exact form
        // for B and P below (Kg, Qg, Kd and gamma are in range either way)
        bool wild = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wild |= !(fabsf(G[j]) <= kSafeGate);
#pragma unroll
            for (int i = 0; i < 4; ++i) wild |= !(fabsf(g[i][j]) <= kSafeGate);
        }
        if (wild) sm.wild = 1;
    }
    // gated keys and queries
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i, c0 = 4 * cg;
        const float kk[4] = {kr4[i].x, kr4[i].y, kr4[i].z, kr4[i].w};
        const float qq[4] = {qr4[i].x, qr4[i].y, qr4[i].z, qr4[i].w};
        f32x4 vkg, vkn, vqg, vkd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float gv = g[i][e];
            const float eg = gate_exp(gv), en = gate_exp(-gv), ed = gate_exp(G[e] - gv);
            vkg[e] = kk[e] * eg;
            vkn[e] = kk[e] * en;
            vqg[e] = qq[e] * eg;
            vkd[e] = kk[e] * ed;
        }
        put4t(sm.kg + r * LDD + c0, vkg);
        put4t(sm.u1.a.kn + r * LDD + c0, vkn);
        put4t(sm.u1.a.qg + r * LDD + c0, vqg);
        put4t(oKd + r * D + c0, vkd);
        put4t(oKg + r * D + c0, vkg);
        put4t(oQg + r * D + c0, scale * vqg);
    }
    __syncthreads();
    if (!sm.wild) {
        // B = Kg Kn^T (fp32) and scale P^T, P = lower(Qg Kn^T)
        mm<4, 4, D, GT>(sm.kg, LDD, sm.u1.a.kn, LDD, [&](int mi, int ni, f32x4 acc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mi + 4 * g4 + i, s = 16 * ni + ln;
                sm.u2.bm[r * (C + 1) + s] = acc[i];
            }
        });
        mm<4, 4, D, GT>(sm.u1.a.qg, LDD, sm.u1.a.kn, LDD, [&](int mi, int ni, f32x4 acc) {
            const int r0 = 16 * mi + 4 * g4, s = 16 * ni + ln;
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = s <= r0 + i ? scale * acc[i] : 0.f;
            put4t(oPt + s * C + r0, x);
        });
    } else if (!sm.pairwise) {
        // The chunk's gates leave the factored form's range (K e^-g
        // overflows) but each 16-row block's own sum stays in it: the decay
        // between rows r and s (s <= r) splits at the cumulative gate rho_I
        // before r's row block I, e^{g_r - g_s} = e^{g_r - rho_I} e^{rho_I - g_s},
        // so B and P are again matrix-core products, of X_I = K_I e^{g - rho_I}
        // (and Q_I e^{g - rho_I}) with Y^(I) = K e^{rho_I - g} over the rows of
        // blocks 0..I; every factor is <= 1 except the second one inside
        // block I, which the block's sum bounds.  Per round of 32 channels
        // thread (rg, cg) stages channel 4 cg + round of its 4 rows as bf16
        // in the dead K e^-g / Q e^g rows; wave w accumulates the 20 lower
        // tiles w, w + 8, w + 16 (B, then P).
        static_assert((2 * C + 160) * BRS * sizeof(uint16_t) <= sizeof(sm.u1.a),
                      "the staged rows fit the dead rows");
        uint16_t* bx = reinterpret_cast<uint16_t*>(&sm.u1.a);
        uint16_t* bqx = bx + C * BRS;
        uint16_t* by = bqx + C * BRS;
        const int wave = tid >> 6, Ir = rg >> 2;
        // rho_1..3 on the thread's channels (read before B overwrites the scan)
        f32x4 rho[3];
#pragma unroll
        for (int I = 0; I < 3; ++I) rho[I] = *reinterpret_cast<const f32x4*>(sm.u2.a.scan + 4 * (I + 1) * D + 4 * cg);
        f32x4 acc[3];
#pragma unroll
        for (int x = 0; x < 3; ++x) acc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int round = 0; round < 4; ++round) {
            if (round > 0) __syncthreads();            // the last round's reads are done
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * rg + i;
                const float kx = f4_at(kr4[i], round), qx = f4_at(qr4[i], round);
                const float gv = g[i][round];
                const float f = gate_exp(gv - (Ir == 0 ? 0.f : rho[Ir - 1][round]));
                bx[r * BRS + cg] = bf(kx * f);
                bqx[r * BRS + cg] = bf(qx * f);
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if (I < Ir) continue;
                    const float rI = I == 0 ? 0.f : rho[I - 1][round];
                    by[(8 * I * (I + 1) + r) * BRS + cg] = bf(kx * gate_exp(rI - gv));
                }
            }
            __syncthreads();
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int t = wave + 8 * x;
                if (t >= 20) continue;
                const int tl = t < 10 ? t : t - 10;
                const int I = (tl >= 1) + (tl >= 3) + (tl >= 6), J = tl - I * (I + 1) / 2;
                const uint16_t* xs = (t < 10 ? bx : bqx) + (16 * I + ln) * BRS + 8 * g4;
                const uint16_t* ys = by + (8 * I * (I + 1) + 16 * J + ln) * BRS + 8 * g4;
                acc[x] = mma32(*reinterpret_cast<const u32x4*>(xs), *reinterpret_cast<const u32x4*>(ys),
                               acc[x]);
            }
        }
        __syncthreads();                       // the staged rows are dead
        float* ptab = reinterpret_cast<float*>(&sm.u1.a);   // P, [C][C + 1]
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int t = wave + 8 * x;
            if (t >= 20) continue;
            const int tl = t < 10 ? t : t - 10;
            const int I = (tl >= 1) + (tl >= 3) + (tl >= 6), J = tl - I * (I + 1) / 2;
            float* tab = t < 10 ? sm.u2.bm : ptab;
#pragma unroll
            for (int i = 0; i < 4; ++i) tab[(16 * I + 4 * g4 + i) * (C + 1) + 16 * J + ln] = acc[x][i];
        }
        __syncthreads();
        for (int idx = tid; idx < C * C; idx += GT) {
            const int s = idx / C, r = idx % C;
            oPt[s * C + r] = bf(s <= r ? scale * ptab[r * (C + 1) + s] : 0.f);
        }
    } else {
        // ... and a 16-row block's own sum leaves it too: B and P entry by
        // entry, each with its own factor e^{g_r - g_s} <= 1 (kda_exact.h),
        // from the raw k, q and gates staged 32 channels at a time in the
        // dead K e^-g / Q e^g rows.
        static_assert(GT == kExactThreads, "one exact unit per thread");
        static_assert(3 * C * kExactXS * sizeof(float) <= sizeof(sm.u1.a) &&
                          C * (C + 1) * sizeof(float) <= sizeof(sm.u1.a),
                      "the staged rows and P fit the dead rows");
        float* sk = reinterpret_cast<float*>(&sm.u1.a);
        float* sq = sk + C * kExactXS;
        float* sg = sq + C * kExactXS;
        const ExactUnit u = exact_unit(tid);
        float a[4][2], pp[4][2];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) a[x][y] = pp[x][y] = 0.f;
#pragma unroll 1
        for (int round = 0; round < 4; ++round) {
            if (round > 0) __syncthreads();
            if ((cg >> 3) == round) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float kk[4] = {kr4[i].x, kr4[i].y, kr4[i].z, kr4[i].w};
                    const float qq[4] = {qr4[i].x, qr4[i].y, qr4[i].z, qr4[i].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int e = (4 * rg + i) * kExactXS + 4 * (cg & 7) + j;
                        sk[e] = kk[j];
                        sq[e] = qq[j];
                        sg[e] = g[i][j];
                    }
                }
            }
            __syncthreads();
            exact_accumulate(u, sk, sq, sg, kLog2e, a, pp);
        }
        exact_reduce(u, a, pp);
        __syncthreads();                       // the staged rows are dead
        float* ptab = sk;                      // P, [C][C + 1]
        if (exact_writer(u, tid)) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) {
                    const int r = 4 * u.bi + x, s = 2 * u.bj + y;
                    if (s < r) sm.u2.bm[r * (C + 1) + s] = a[x][y];
                    if (s <= r) ptab[r * (C + 1) + s] = pp[x][y];
                }
        }
        __syncthreads();
        for (int idx = tid; idx < C * C; idx += GT) {
            const int s = idx / C, r = idx % C;
            oPt[s * C + r] = bf(s <= r ? scale * ptab[r * (C + 1) + s] : 0.f);
        }
    }
    __syncthreads();
    // Minv = (I + A)^-1, A = strict_lower(Diag(beta) B), blockwise in 16x16
    // blocks.  The diagonal blocks (unit lower triangular) by forward
    // substitution, one thread per column with the column in registers;
    // then block row I = 1..3 from the rows above it:
    //     Minv_IJ = -Minv_II sum_{K=J}^{I-1} A_IK Minv_KJ     (J < I)
    // on fp32 matrix cores (16x16x4), wave J computing block (I, J).
    if (tid < C) {
        const int col = tid, base = col & ~15;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int r = base + rr;
            float acc = 0.f;
#pragma unroll
            for (int ss = 0; ss < rr; ++ss) acc += sm.u2.bm[r * (C + 1) + base + ss] * x[ss];
            x[rr] = (r == col ? 1.f : 0.f) - sm.bs[r] * acc;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sm.u1.b.mi[(base + rr) * (C + 1) + col] = x[rr];
        for (int r = 0; r < base; ++r) sm.u1.b.mi[r * (C + 1) + col] = 0.f;
    }
    __syncthreads();
    for (int I = 1; I < 4; ++I) {
        const int J = tid >> 6;
        if (J < I) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int row = 16 * I + ln;
            for (int K = J; K < I; ++K) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int kc = 16 * K + 4 * kk + g4;
                    const float a = sm.bs[row] * sm.u2.bm[row * (C + 1) + kc];
                    const float b = sm.u1.b.mi[kc * (C + 1) + 16 * J + ln];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
                }
            }
            float* xs = sm.u1.b.xs[J];
#pragma unroll
            for (int i = 0; i < 4; ++i) xs[(4 * g4 + i) * 17 + ln] = acc[i];
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float a = sm.u1.b.mi[row * (C + 1) + 16 * I + 4 * kk + g4];
                const float b = xs[(4 * kk + g4) * 17 + ln];
                m = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, m, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.u1.b.mi[(16 * I + 4 * g4 + i) * (C + 1) + 16 * J + ln] = -m[i];
        }
        __syncthreads();
    }
    for (int idx = tid; idx < C * C; idx += GT) {
        const int r = idx / C, s = idx % C;
        const float m = sm.u1.b.mi[r * (C + 1) + s];
        oMinv[idx] = m;
        sm.u1.b.tt[r * LDC + s] = bf(m * sm.bs[s]);     // T = Minv Diag(beta)
    }
    __syncthreads();
    // -W^T, W = T Kg (Kg read by rows of K)
    mm<4, 8, C, GT, kKc, kMc>(sm.u1.b.tt, LDC, sm.kg, LDD, [&](int mi, int ni, f32x4 acc) {
        put4t(oWt + (16 * ni + ln) * C + 16 * mi + 4 * g4, -acc);
    });
}

// ===================================================================
// carry: dS backwards through the chunks of one block
// ===================================================================
struct alignas(16) CarryLds {
    bf16_t kd[C * LDD];
    bf16_t pt[C * LDC];
    bf16_t qg[C * LDD];                // scale Qg
    bf16_t wt[D * LDC];
    float gam[D];
    bf16_t dol[C * LDO];               // dO of the tile's columns
    bf16_t dst[kCarryTile / 16][16 * LDD];   // each 16-column slab of dS, transposed
    bf16_t det[kCarryTile / 16][16 * LDC];   // each 16-column slab of dE, transposed
};

// copy a [rows][cols] bf16 matrix (global, contiguous) into LDS rows of ld
template <int NTH = NT>
__device__ __forceinline__ void copy_rows(bf16_t* dst, int ld, const bf16_t* src, int rows,
                                          int cols) {
    const int per = cols / 8;
    for (int u = threadIdx.x; u < rows * per; u += NTH) {
        const int r = u / per, x = (u % per) * 8;
        *reinterpret_cast<u32x4*>(dst + r * ld + x) = *reinterpret_cast<const u32x4*>(src + r * cols + x);
    }
}

__global__ __launch_bounds__(GG)
void bwd_carry_kernel(const uint8_t* __restrict__ slots, const bf16_t* __restrict__ dO,
                      const int32_t* __restrict__ cu, int N, int H, int c_lo, int L_b, int c_end,
                      float* __restrict__ dstate, bf16_t* __restrict__ dsblk,
                      bf16_t* __restrict__ deblk, float* __restrict__ dh0)
{
    __shared__ CarryLds sm;
    constexpr int R = D / kCarryTile;
    const int pair = blockIdx.x / R, tile = blockIdx.x % R;
    const int n = pair / H, h = pair % H;
    if (n >= N) return;            // the grid is exactly N * H * R work-groups
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, ln = lane & 15;
    // 16 waves: wave w owns value columns 16 (w % NS) .. +15 of the tile,
    // key rows RW (w / NS) .. +RW-1 of the state and row tiles
    // ME (w / NS) .. +ME-1 of dE
    constexpr int NS = kCarryTile / 16, NQ = 16 / NS, RW = D / NQ, MS = RW / 16, ME = C / 16 / NQ;
    static_assert(NS * NQ == GG / 64 && ME >= 1, "the wave map");
    const int slab = wave % NS, quarter = wave / NS;
    const int64_t t_begin = cu[n], t_end = cu[n + 1];
    const int nch = static_cast<int>((t_end - t_begin + C - 1) / C);
    const int hi = min(nch, c_lo + L_b) - 1;          // last chunk of this block
    const int jc = tile * kCarryTile + 16 * slab + ln; // this lane's value column
    const int rb = RW * quarter;                       // this wave's first key row
    float* st = dstate + (static_cast<int64_t>(n) * H + h) * kState;
    if (hi < c_lo) {
        // no chunk here; an empty sequence still gets dh0 = dhT (or zeros)
        if (c_lo == 0 && dh0) {
            float* d0 = dh0 + (static_cast<int64_t>(n) * H + h) * kState;
            for (int e = tid; e < D * kCarryTile; e += GG) {
                const int row = e / kCarryTile, col = tile * kCarryTile + e % kCarryTile;
                d0[row * D + col] = st[row * D + col];
            }
        }
        return;
    }
    // dS slab: S[m][i] = dS[rb + 16m + 4g + i][jc]
    f32x4 S[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[m][i] = st[(rb + 16 * m + 4 * g4 + i) * D + jc];

    // The next chunk's operands load into registers while this chunk
    // computes.  Kd, P^T, Qg and W^T are 3584 16-byte units (Kd, then P^T,
    // Qg and W^T contiguous from kOffPt): unit x * 1024 + tid, x < 4, for
    // the units that exist; dO's 64-row tile is C * kCarryTile / 8 more,
    // one per thread of the first ones.
    constexpr int NUNIT = (C * D + C * C + 2 * D * C) / 8;
    constexpr int PER = (NUNIT + GG - 1) / GG;
    constexpr int DOU = C * kCarryTile / 8, DOP = kCarryTile / 8;
    static_assert(NUNIT == 3584 && PER == 4 && DOU <= GG, "the unit map below");
    u32x4 pre[PER], pdo = {0u, 0u, 0u, 0u};
    float pgam = 0.f;
    auto fetch = [&](int j) {
        const int64_t slot = (static_cast<int64_t>(n) * L_b + (j - c_lo)) * H + h;
        const uint8_t* sp = slots + slot * static_cast<int64_t>(kSlot);
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = x * GG + tid;
            const int byte = u < C * D / 8 ? 16 * u : kOffPt + 16 * (u - C * D / 8);
            if (u < NUNIT) pre[x] = *reinterpret_cast<const u32x4*>(sp + byte);
        }
        if (tid < D) pgam = reinterpret_cast<const float*>(sp + kOffGam)[tid];
        if (tid < DOU) {
            const int64_t t0 = t_begin + static_cast<int64_t>(j) * C;
            const int len = static_cast<int>(min<int64_t>(C, t_end - t0));
            const int r = tid / DOP, part = tid % DOP;
            pdo = *reinterpret_cast<const u32x4*>(dO + ((t0 + min(r, len - 1)) * H + h) * D +
                                                  tile * kCarryTile + 8 * part);
            if (r >= len) pdo = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = x * GG + tid;
            if (u >= NUNIT) continue;
            bf16_t* dst;
            if (u < C * D / 8) {
                dst = sm.kd + (u / 16) * LDD + (u % 16) * 8;
            } else if (u < C * D / 8 + C * C / 8) {
                const int w = u - C * D / 8;
                dst = sm.pt + (w / 8) * LDC + (w % 8) * 8;
            } else if (u < 2 * C * D / 8 + C * C / 8) {
                const int w = u - C * D / 8 - C * C / 8;
                dst = sm.qg + (w / 16) * LDD + (w % 16) * 8;
            } else {
                const int w = u - 2 * C * D / 8 - C * C / 8;
                dst = sm.wt + (w / 8) * LDC + (w % 8) * 8;
            }
            *reinterpret_cast<u32x4*>(dst) = pre[x];
        }
        if (tid < D) sm.gam[tid] = pgam;
        if (tid < DOU) {
            const int r = tid / DOP, part = tid % DOP;
            *reinterpret_cast<u32x4*>(sm.dol + r * LDO + 8 * part) = pdo;
        }
    };

    fetch(hi);
    for (int j = hi; j >= c_lo; --j) {
        const int64_t slot = (static_cast<int64_t>(n) * L_b + (j - c_lo)) * H + h;
        put();
        // dS' of this chunk (bf16, for the grad pass) and as a bf16 B operand
        bf16_t* dsp = dsblk + slot * kState;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dsp[(rb + 16 * m + 4 * g4 + i) * D + jc] = bf(S[m][i]);
            put4t(&sm.dst[slab][ln * LDD + rb + 16 * m + 4 * g4], S[m]);
        }
        __syncthreads();
        if (j > c_lo) fetch(j - 1);
        // dE = Kd dS' + scale P^T dO  (this slab's 16 columns, this wave's row tiles)
        bf16_t* dep = deblk + slot * (static_cast<int64_t>(C) * D);
        const bf16_t* dsw = sm.dst[slab];
        const bf16_t* dow = sm.dol + 16 * slab;   // dO by rows of K
#pragma unroll
        for (int me = 0; me < ME; ++me) {
            const int m = ME * quarter + me;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mm<D>(sm.kd + 16 * m * LDD, LDD, dsw, LDD, lane, acc);
            acc = tile_mm<C, kKc, kMc>(sm.pt + 16 * m * LDC, LDC, dow, LDO, lane, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) dep[(16 * m + 4 * g4 + i) * D + jc] = bf(acc[i]);
            put4t(&sm.det[slab][ln * LDC + 16 * m + 4 * g4], acc);
        }
        __syncthreads();
        // dS = Diag(gamma) dS' + scale Qg^T dO - W^T dE  (this wave's key rows)
        const bf16_t* dew = sm.det[slab];
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int mb = MS * quarter + m;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = sm.gam[16 * mb + 4 * g4 + i] * S[m][i];
            acc = tile_mm<C, kMc, kMc>(sm.qg + 16 * mb, LDD, dow, LDO, lane, acc);
            acc = tile_mm<C>(sm.wt + 16 * mb * LDC, LDC, dew, LDC, lane, acc);
            S[m] = acc;
        }
        __syncthreads();
    }
    float* dst_out = c_lo == 0 ? dh0 : st;
    // a sequence longer than the call's chunk bound (the caller's
    // max_seqlen) was cut short: dh0 is NaN, not a silently wrong adjoint
    const bool cut = c_lo == 0 && nch > c_end;
    if (dst_out) {
        dst_out += c_lo == 0 ? (static_cast<int64_t>(n) * H + h) * kState : 0;
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst_out[(rb + 16 * m + 4 * g4 + i) * D + jc] = cut ? __builtin_nanf("") : S[m][i];
    }
}

// ===================================================================
// grad: one work-group per (chunk, head).  Phase A takes the products with
// the chunk's start state and its adjoints; the terms phase B needs stay in
// registers (dKg_W, dQg_S, dKd, dT, dP: each wave keeps the 16x16 tiles it
// computed, and phase B hands the same tiles to the same waves); phase B
// then solves the triangular-system and gate terms and writes dq, dk,
// dlog_alpha and dbeta.  The two phases share the LDS.  Every matrix is
// staged once, in the layout it arrives in; a product that contracts over
// the contiguous index of an operand reads it with 16-byte reads, one that
// contracts over its rows with transpose reads (kMc).
// ===================================================================
constexpr int LDT = D + 16;    // rows read only by transpose reads: a row step of 8 banks
constexpr int LDG = D + 4;     // fp32 row stride of the gates: rows 4 banks apart, so 16
                               // lanes reading one channel of 16 rows hit 16 banks

struct alignas(16) GradALds {
    bf16_t st[D * LDD];        // S^T [value j][key c] (the recorded layout)
    bf16_t dsl[D * LDD];       // dS' [key c][value j]
    bf16_t kg[C * LDD];        // Kg; later E
    bf16_t r[C * LDD];         // V, then R; later dV
    bf16_t de[C * LDD];        // dE
    bf16_t dol[C * LDD];       // dO
    bf16_t mvb[C * LDC];       // Minv Diag(beta)
    float bs[C];
    float dgp[GG / D][D];      // dgamma over eight parts of the value columns
};
struct alignas(16) GradBLds {
    float g[C * LDG];          // cumulative gates
    bf16_t kg[C * LDT], kn[C * LDT], qg[C * LDT];   // gated keys and queries, row-major
    bf16_t mv[C * LDC];        // Minv
    bf16_t dp[C * LDC];        // dP
    bf16_t yt[C * LDC];        // (dT Diag(beta))^T; later dB
    bf16_t z[C * LDC];         // Z = Minv^T dT Diag(beta)
    float bs[C];
    float db[C];               // dbeta
    float dbp[4][C];           // dbeta_A per 16-column block, summed in order
    float hp[D / 16][C];       // per-head gate: dlog_alpha per channel block
    float ftot[4][D];          // dlog_alpha: per row block and channel, the sum of dg
    float fdg[2][D];           // ... and the two halves of dG's sum over the rows
    float gscan[(C / 4) * D];  // the gate scan over row groups
    float gtot[D];
};
union alignas(16) GradLds {
    GradALds a;
    GradBLds b;
};

// fp32 [rows][D] global (null = zeros) -> bf16 LDS, transposed (row = column index)
template <int NTH = NT>
__device__ __forceinline__ void stage_f32_t(const float* src, int rows, bf16_t* tr, int ldt) {
    for (int u = threadIdx.x; u < rows * (D / 4); u += NTH) {
        const int r = u / (D / 4), c0 = (u % (D / 4)) * 4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (src) x = *reinterpret_cast<const f32x4*>(src + r * D + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) tr[(c0 + e) * ldt + r] = bf(x[e]);
    }
}

// the start state of chunk j of sequence n: for the first chunk h0 (fp32;
// null = zeros), else the state the forward pass recorded after chunk j-1
// (bf16, transposed: [value column][key row])
__device__ __forceinline__ const bf16_t* recorded_state(const ChunkRef& c, const bf16_t* sall,
                                                        const int32_t* cu, int H) {
    const int64_t idx = c.n + cu[c.n] / C + (c.j - 1);
    return sall + (idx * H + c.h) * kState;
}

template <typename T, int GATE>
__global__ __launch_bounds__(GG)
void bwd_grad_kernel(const uint8_t* __restrict__ slots, const bf16_t* __restrict__ dsblk,
                     const bf16_t* __restrict__ deblk, const bf16_t* __restrict__ sall,
                     const float* __restrict__ h0, const T* __restrict__ q,
                     const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dO,
                     const float* __restrict__ la, const float* __restrict__ beta,
                     const int32_t* __restrict__ cu, int H, int c_lo, int L_b, float scale,
                     T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
                     float* __restrict__ dla, float* __restrict__ dbeta)
{
    __shared__ GradLds sm_u;
    __shared__ float s_dgam[D], s_dbT[4][C];   // phase A -> phase B
    __shared__ int s_wild;                     // the chunk is beyond the factored range ...
    __shared__ int s_pair;                     // ... and a 16-row block's own gate sum too
    ChunkRef c;
    if (!chunk_of(blockIdx.x, H, c_lo, L_b, cu, c)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, ln = lane & 15;
    if (tid == 0) s_wild = s_pair = 0;
    const uint8_t* sp = slots + c.slot * static_cast<int64_t>(kSlot);
    const float* mvg = reinterpret_cast<const float*>(sp + kOffMinv);
    const float* S0f = c.j == 0 && h0 ? h0 + (static_cast<int64_t>(c.n) * H + c.h) * kState
                                      : nullptr;

    // tiles kept in registers (tile x of this wave is t = wave + 16x):
    // [C][D] terms, 4 x 8 tiles: row blocks wave / 8 + 2x, column block
    // wave % 8; [C][C] terms, 4 x 4 tiles: row block wave / 4, column block
    // wave % 4
    f32x4 rKgW[2], rQgS[2], rKd[2];
    f32x4 rT[1], rP[1];
    // fp32 Minv, loaded with the first round and used later: the row this
    // thread stages (twice), and the entries of this wave's dT tile (row
    // 16 (wave / 4) + 4 g4 + i, column s2) for dbeta_T
    f32x4 mvr;
    float mvd[4];
    // phase B's inputs load with phase A's: this thread's block of k and q
    // (raw bf16 pairs) and of raw gates, and beta (threads past the 512
    // blocks of the chunk hold zeros and load nothing)
    static_assert(sizeof(T) == 2, "bf16 inputs");
    u32x2 kraw[4], qraw[4];
    f32x4 graw[4];
    float bsv;
    load_rows4_raw(reinterpret_cast<const bf16_t*>(k), c, H, kraw);
    load_rows4_raw(reinterpret_cast<const bf16_t*>(q), c, H, qraw);
    load_gate_block<GATE>(la, beta, c, H, graw, bsv);
    {
        const int s2 = 16 * (wave % 4) + ln, mi = wave / 4;
        mvr = *reinterpret_cast<const f32x4*>(mvg + (tid / (C / 4)) * C + 4 * (tid % (C / 4)));
#pragma unroll
        for (int i = 0; i < 4; ++i) mvd[i] = mvg[(16 * mi + 4 * g4 + i) * C + s2];
    }
    // =========================== phase A ===========================
    {
        GradALds& sm = sm_u.a;
        // ---- one round of loads, each matrix in its own layout: S^T, dS',
        //      Kg, V, dE, dO, beta, Minv Diag(beta)
        if (c.j == 0) stage_f32_t<GG>(S0f, D, sm.st, LDD);
        else copy_rows<GG>(sm.st, LDD, recorded_state(c, sall, cu, H), D, D);
        copy_rows<GG>(sm.dsl, LDD, dsblk + c.slot * kState, D, D);
        copy_rows<GG>(sm.kg, LDD, reinterpret_cast<const bf16_t*>(sp + kOffKg), C, D);
        copy_rows<GG>(sm.de, LDD, deblk + c.slot * (static_cast<int64_t>(C) * D), C, D);
        for (int u = tid; u < C * (D / 8); u += GG) {
            const int r = u / (D / 8), c8 = (u % (D / 8)) * 8;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (r < c.len) x = *reinterpret_cast<const u32x4*>(dO + ((c.t0 + r) * H + c.h) * D + c8);
            *reinterpret_cast<u32x4*>(sm.dol + r * LDD + c8) = x;
        }
        for (int u = tid; u < C * (D / 4); u += GG) {
            const int r = u / (D / 4), c0 = (u % (D / 4)) * 4;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < c.len) x = elem<T>::load4(v + ((c.t0 + r) * H + c.h) * D + c0);
            put4t(sm.r + r * LDD + c0, f32x4{x.x, x.y, x.z, x.w});
        }
        if (tid < C) sm.bs[tid] = tid < c.len ? beta[(c.t0 + tid) * H + c.h] : 0.f;
        __syncthreads();
        {
            const int r = tid / (C / 4), s0 = (tid % (C / 4)) * 4;
            put4t(sm.mvb + r * LDC + s0, f32x4{mvr[0] * sm.bs[s0], mvr[1] * sm.bs[s0 + 1],
                                               mvr[2] * sm.bs[s0 + 2], mvr[3] * sm.bs[s0 + 3]});
        }
        // ---- R = V - Kg S (B = S^T rows)
        mm<4, 8, D, GG>(sm.kg, LDD, sm.st, LDD, [&](int mi, int ni, f32x4 acc) {
            const int r0 = 16 * mi + 4 * g4, col = 16 * ni + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16_t* p = sm.r + (r0 + i) * LDD + col;
                *p = bf(bf16_to_f32(*p) - acc[i]);
            }
        });
        // ---- dgamma = rowsum(dS' . S) from the bf16 records, summed in fp32:
        //      thread (part, key c) takes value columns 16 part .. +15
        {
            const int ch = tid & (D - 1), part = tid >> 7;
            float acc = 0.f;
#pragma unroll
            for (int x = 0; x < 16; x += 8) {
                const int j0 = 16 * part + x;
                const u32x4 dw = *reinterpret_cast<const u32x4*>(sm.dsl + ch * LDD + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc += lo_bf(dw[e]) * bf16_to_f32(sm.st[(j0 + 2 * e) * LDD + ch]) +
                           hi_bf(dw[e]) * bf16_to_f32(sm.st[(j0 + 2 * e + 1) * LDD + ch]);
            }
            sm.dgp[part][ch] = acc;
        }
        __syncthreads();
        // ---- E = (Minv Diag(beta)) R over Kg (R read by rows of K)
        bf16_t* E = sm.kg;
        mm<4, 8, C, GG, kKc, kMc>(sm.mvb, LDC, sm.r, LDD, [&](int mi, int ni, f32x4 acc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) E[(16 * mi + 4 * g4 + i) * LDD + 16 * ni + ln] = bf(acc[i]);
        });
        // ---- dT = dE R^T (kept), dbeta_T = diag(Minv^T dT): wave w holds
        //      the tile (row block w / 4, column block w % 4)
        mm_regs<4, D, 1, GG>(sm.de, LDD, sm.r, LDD, rT);
        {
            const int s2 = 16 * (wave % 4) + ln;
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) part += mvd[i] * rT[0][i];
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            if (g4 == 0) s_dbT[wave / 4][s2] = part;
        }
        if (tid < D) {
            float acc = 0.f;
#pragma unroll
            for (int p = 0; p < GG / D; ++p) acc += sm.dgp[p][tid];
            s_dgam[tid] = acc;
        }
        __syncthreads();
        // ---- dV = T^T dE = (Minv Diag(beta))^T dE (over R; both operands by rows of K)
        bf16_t* dV = sm.r;
        mm<4, 8, C, GG, kMc, kMc>(sm.mvb, LDC, sm.de, LDD, [&](int mi, int ni, f32x4 acc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dV[(16 * mi + 4 * g4 + i) * LDD + 16 * ni + ln] = bf(acc[i]);
        });
        __syncthreads();
        // dV out in whole 16-byte pieces of its rows (dv takes the bf16 of
        // the same value the products below use)
        static_assert(sizeof(T) == 2 && C * D / 8 == GG, "one 16-byte piece of dV per thread");
        {
            const int r = tid / (D / 8), c8 = (tid % (D / 8)) * 8;
            if (r < c.len)
                *reinterpret_cast<u32x4*>(dv + ((c.t0 + r) * H + c.h) * D + c8) =
                    *reinterpret_cast<const u32x4*>(dV + r * LDD + c8);
        }
        // ---- dKg_W = -dV S^T, dQg_S = scale dO S^T (kept; S^T read by rows of K)
        mm_regs<8, D, 2, GG, kKc, kMc>(dV, LDD, sm.st, LDD, rKgW);
        mm_regs<8, D, 2, GG, kKc, kMc>(sm.dol, LDD, sm.st, LDD, rQgS);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            rKgW[x] = -rKgW[x];
            rQgS[x] = scale * rQgS[x];
        }
        // ---- dKd = E dS'^T, dP = lower(scale dO E^T) (kept)
        mm_regs<8, D, 2, GG>(E, LDD, sm.dsl, LDD, rKd);
        mm_regs<4, D, 1, GG>(sm.dol, LDD, E, LDD, rP);
        {
            const int mi = wave / 4, ni = wave % 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mi + 4 * g4 + i, s2 = 16 * ni + ln;
                rP[0][i] = s2 <= r ? scale * rP[0][i] : 0.f;
            }
        }
        __syncthreads();   // phase B reuses the LDS
    }
    // =========================== phase B ===========================
    GradBLds& sm = sm_u.b;
    // Minv into LDS; the gates scanned as in the prep (the same gate bits)
    put4t(sm.mv + (tid / (C / 4)) * LDC + 4 * (tid % (C / 4)), mvr);
    {
        float gr[4][4];
        f32x4 Gr;
        scan_gate_block(graw, bsv, sm.gscan, sm.gtot, sm.bs, gr, Gr);
        if (tid < GT) {
            bool wild = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wild |= !(fabsf(Gr[j]) <= kSafeGate);
#pragma unroll
                for (int i = 0; i < 4; ++i) wild |= !(fabsf(gr[i][j]) <= kSafeGate);
            }
            if (wild) s_wild = 1;
        }
        if (tid < D) {
            // the gate sums of the four 16-row blocks on channel tid
            const float r1 = sm.gscan[4 * D + tid], r2 = sm.gscan[8 * D + tid];
            const float r3 = sm.gscan[12 * D + tid], gt = sm.gtot[tid];
            const bool far = !(fabsf(r1) <= kSafeGate && fabsf(r2 - r1) <= kSafeGate &&
                               fabsf(r3 - r2) <= kSafeGate && fabsf(gt - r3) <= kSafeGate);
            if (far) s_pair = 1;
        }
        // the gates for the final tiles, and the gated keys and queries
        // (one thread per 4 x 4 block of the chunk)
        if (tid < GT) {
            const int rg = tid >> 5, c0 = 4 * (tid & 31);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * rg + i;
                *reinterpret_cast<f32x4*>(sm.g + r * LDG + c0) = f32x4{gr[i][0], gr[i][1], gr[i][2], gr[i][3]};
                const float kk[4] = {lo_bf(kraw[i][0]), hi_bf(kraw[i][0]), lo_bf(kraw[i][1]),
                                     hi_bf(kraw[i][1])};
                const float qq[4] = {lo_bf(qraw[i][0]), hi_bf(qraw[i][0]), lo_bf(qraw[i][1]),
                                     hi_bf(qraw[i][1])};
                f32x4 kg, kn, qg;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float eg = gate_exp(gr[i][e]), en = gate_exp(-gr[i][e]);
                    kg[e] = kk[e] * eg;
                    kn[e] = kk[e] * en;
                    qg[e] = qq[e] * eg;
                }
                put4t(sm.kg + r * LDT + c0, kg);
                put4t(sm.kn + r * LDT + c0, kn);
                put4t(sm.qg + r * LDT + c0, qg);
            }
        }
    }
    // the final tiles of this wave: key channel block cb, row blocks
    // wave / 8 + 2x (the tiles of rKgW, rQgS, rKd); k and q at those
    // positions, loaded here and used after the triangular-system products
    const int cb = wave % 8, ch = 16 * cb + ln;
    float kv[2][4], qv[2][4];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * (wave / 8 + 2 * x) + 4 * g4 + i;
            const int rr = min(r, c.len - 1);        // rows past the chunk: any valid row
            const int64_t row = ((c.t0 + rr) * H + c.h) * D + ch;
            kv[x][i] = elem<T>::load(k + row);
            qv[x][i] = elem<T>::load(q + row);
        }
    // (dT Diag(beta))^T and dP from this wave's dT and dP tiles
    {
        const int mi = wave / 4, s2 = 16 * (wave % 4) + ln;
        put4t(sm.yt + s2 * LDC + 16 * mi + 4 * g4, sm.bs[s2] * rT[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.dp[(16 * mi + 4 * g4 + i) * LDC + s2] = bf(rP[0][i]);
    }
    if (tid < C) sm.db[tid] = (s_dbT[0][tid] + s_dbT[1][tid]) + (s_dbT[2][tid] + s_dbT[3][tid]);
    __syncthreads();
    // A chunk whose gates leave the factored form's range takes the exact
    // form (kda_exact.h): its B and the products with dB and dP are summed
    // pair by pair with factors e^{g_r - g_s} <= 1, from the raw k and q,
    // which replace the gated copies in LDS
    const bool exact = s_wild != 0;
    if (exact) {
        if (tid < GT) {
            const int rg = tid >> 5, c0 = 4 * (tid & 31);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * rg + i;
                put4t(sm.kn + r * LDT + c0, f32x4{lo_bf(kraw[i][0]), hi_bf(kraw[i][0]),
                                                  lo_bf(kraw[i][1]), hi_bf(kraw[i][1])});
                put4t(sm.qg + r * LDT + c0, f32x4{lo_bf(qraw[i][0]), hi_bf(qraw[i][0]),
                                                  lo_bf(qraw[i][1]), hi_bf(qraw[i][1])});
            }
        }
        __syncthreads();
    }
    // B = Kg Kn^T at this wave's dA tile (for dbeta_A; the prep's inverse
    // used the same bf16 operands and product order, or the same form beyond
    // the factored range)
    f32x4 bmt[1];
    if (!exact) {
        mm_regs<4, D, 1, GG>(sm.kg, LDT, sm.kn, LDT, bmt);
    } else if (!s_pair) {
        // the prep's blocked form: per round j, X = K e^{g - rho_I} and the
        // Y^(I) = K e^{rho_I - g} of channels 4 c + j at column c, bf16, from
        // the same gate bits (rho_I: the scan's prefix before row block I),
        // in the dead gated-key rows; thread (r, cp) stages row r, columns
        // 2 cp and 2 cp + 1
        static_assert((C + 160) * BRS <= C * LDT && GG == C * 16, "the staged rows; one row per 16 threads");
        uint16_t* bx = sm.kg;
        uint16_t* by = sm.kg + C * BRS;
        // lane coordinates as opaque values: no address of this rare branch
        // is hoisted to where it would hold registers on the common path
        int r = tid >> 4, cp = tid & 15, w = wave, l16 = ln, gq = g4;
        asm volatile("" : "+v"(r), "+v"(cp), "+v"(w), "+v"(l16), "+v"(gq));
        const int Ir = r >> 4, mi = w / 4, ni = w % 4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int round = 0; round < 4; ++round) {
            if (round > 0) __syncthreads();            // the last round's reads are done
#pragma unroll 1
            for (int e = 0; e < 2; ++e) {
                const int col = 2 * cp + e, ch = 4 * col + round;
                const float kx = bf16_to_f32(sm.kn[r * LDT + ch]);
                const float gv = sm.g[r * LDG + ch];
                const float ref = Ir == 0 ? 0.f : sm.gscan[4 * Ir * D + ch];
                bx[r * BRS + col] = bf(kx * gate_exp(gv - ref));
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if (I < Ir) continue;
                    const float rI = I == 0 ? 0.f : sm.gscan[4 * I * D + ch];
                    by[(8 * I * (I + 1) + r) * BRS + col] = bf(kx * gate_exp(rI - gv));
                }
            }
            __syncthreads();
            if (ni <= mi)
                acc = mma32(*reinterpret_cast<const u32x4*>(bx + (16 * mi + l16) * BRS + 8 * gq),
                            *reinterpret_cast<const u32x4*>(by + (8 * mi * (mi + 1) + 16 * ni + l16) * BRS + 8 * gq),
                            acc);
        }
        bmt[0] = acc;
    } else {
        const int mi = wave / 4, s = 16 * (wave % 4) + ln;
        bmt[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int c2 = 0; c2 < D; ++c2) {
            const float ks = bf16_to_f32(sm.kn[s * LDT + c2]), gs = sm.g[s * LDG + c2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mi + 4 * g4 + i;
                const float e = __builtin_amdgcn_exp2f((sm.g[r * LDG + c2] - gs) * kLog2e);
                bmt[0][i] += s < r ? bf16_to_f32(sm.kn[r * LDT + c2]) * ks * e : 0.f;
            }
        }
    }
    // Z = Minv^T (dT Diag(beta))  (Minv read by rows of K)
    mm<4, 4, C, GG, kMc, kKc>(sm.mv, LDC, sm.yt, LDC, [&](int mi, int ni, f32x4 acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.z[(16 * mi + 4 * g4 + i) * LDC + 16 * ni + ln] = bf(acc[i]);
    });
    __syncthreads();
    // dA = -strict_lower(Z Minv^T); dB = Diag(beta) dA over (dT Diag(beta))^T,
    // which nothing reads any more
    {
        f32x4 dA[1];
        mm_regs<4, C, 1, GG>(sm.z, LDC, sm.mv, LDC, dA);
        const int mi = wave / 4, ni = wave % 4;
        const int r0 = 16 * mi + 4 * g4, s2 = 16 * ni + ln;
        float rowpart[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + i;
            const float a = s2 < r ? -dA[0][i] : 0.f;
            rowpart[i] = a * bmt[0][i];                  // dbeta_A
            sm.yt[r * LDC + s2] = bf(sm.bs[r] * a);      // dB = Diag(beta) dA
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float pp = rowpart[i];
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) pp += __shfl_xor(pp, m);
            if (ln == 0) sm.dbp[ni][r0 + i] = pp;
        }
    }
    __syncthreads();
    const bf16_t* dB = sm.yt;
    if (tid >= GG - C) {
        const int r = tid - (GG - C);
        if (r < c.len)
            dbeta[(c.t0 + r) * H + c.h] = sm.db[r] + ((sm.dbp[0][r] + sm.dbp[1][r]) +
                                                      (sm.dbp[2][r] + sm.dbp[3][r]));
    }
    // per 16x16 tile of (row r, key channel c): dKg = dKg_W + dB Kn,
    // dKn = dP^T Qg + dB^T Kg, dQg = dQg_S + dP Kn, then the gate chain;
    // the B fragments of Kn, Kg and Qg (read by rows of K) serve both of
    // the wave's tiles
    const float G = sm.g[(c.len - 1) * LDG + ch];
    float dgr[2][4];          // dg of rows 16 mi + 4 g4 + i, this lane's channel
    float dGp = 0.f;
    if (!exact) {
        u32x4 fkn[2], fkg[2], fqg[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            fkn[s2] = frag<kMc>(sm.kn + 16 * cb, LDT, 32 * s2, lane);
            fkg[s2] = frag<kMc>(sm.kg + 16 * cb, LDT, 32 * s2, lane);
            fqg[s2] = frag<kMc>(sm.qg + 16 * cb, LDT, 32 * s2, lane);
        }
        // every wave holds its fragments of the gated keys and queries:
        // their buffers take dk and dq, which leave in whole 16-byte pieces
        // of rows
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int mi = wave / 8 + 2 * x;
            f32x4 aKg = {0.f, 0.f, 0.f, 0.f}, aKn = aKg, aQg = aKg;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                aKg = mma32(frag<kKc>(dB + 16 * mi * LDC, LDC, 32 * s2, lane), fkn[s2], aKg);
                aKn = mma32(frag<kMc>(dB + 16 * mi, LDC, 32 * s2, lane), fkg[s2], aKn);
                aKn = mma32(frag<kMc>(sm.dp + 16 * mi, LDC, 32 * s2, lane), fqg[s2], aKn);
                aQg = mma32(frag<kKc>(sm.dp + 16 * mi * LDC, LDC, 32 * s2, lane), fkn[s2], aQg);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mi + 4 * g4 + i;
                float dgv = 0.f;
                if (r < c.len) {
                    const float gv = sm.g[r * LDG + ch];
                    const float eg = gate_exp(gv), en = gate_exp(-gv), ed = gate_exp(G - gv);
                    const float dKg = aKg[i] + rKgW[x][i];
                    const float dQg = aQg[i] + rQgS[x][i];
                    const float dKn = aKn[i];
                    const float dKd = rKd[x][i];
                    const float Kg = kv[x][i] * eg, Kn = kv[x][i] * en, Qg = qv[x][i] * eg;
                    const float Kd = kv[x][i] * ed;
                    sm.kg[r * LDT + ch] = bf(dKg * eg + dKn * en + dKd * ed);   // dk
                    sm.kn[r * LDT + ch] = bf(dQg * eg);                         // dq
                    dgv = dKg * Kg - dKn * Kn + dQg * Qg - dKd * Kd;
                    dGp += dKd * Kd;
                }
                dgr[x][i] = dgv;
            }
        }
    } else {
        // per row r and this lane's channel c, with E(r, s) = e^{g_r[c] - g_s[c]}:
        //   FK = sum_{s<r} dB[r][s] k_s E(r, s)     (= (dB Kn)[r] e^{g_r})
        //   FQ = sum_{s<=r} dP[r][s] k_s E(r, s)    (= (dP Kn)[r] e^{g_r})
        //   GS = sum_{r'>r} dB[r'][r] k_r' E(r', r) + sum_{r'>=r} dP[r'][r] q_r' E(r', r)
        //                                           (= (dB^T Kg + dP^T Qg)[r] e^{-g_r})
        // then the chain of the common path with those in place of its
        // products: dk = FK + GS + ..., dq = FQ + ..., dg = FK k + FQ q - GS k + ...
        // dk and dq of each row wait in registers (bf16 pairs) until every
        // wave has read the raw keys and queries
        uint32_t dkq[2][4];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int mi = wave / 8 + 2 * x;
            float gr4[4], fk[4], fq[4], gsum[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gr4[i] = sm.g[(16 * mi + 4 * g4 + i) * LDG + ch];
                fk[i] = fq[i] = gsum[i] = 0.f;
            }
            if (!s_pair) {
                // blocked form: with rho_I the gate before row block I (this
                // lane's channel) and the rows r of block mi,
                //   FK, FQ = e^{g_r - rho_mi} (dB, dP)[r, :] Y,  Y[s] = k_s e^{rho_mi - g_s}
                //     over the rows s of blocks 0..mi (zero beyond);
                //   GS = sum_{I >= mi} e^{rho_I - g_r} (dB_{I,mi}^T X_I + dP_{I,mi}^T QX_I),
                //     X_I[r'] = k_r' e^{g_r' - rho_I}, QX_I with q, r' in block I.
                // Every factor is <= 1 except those inside one row block, which
                // the block's gate sum bounds.  Each lane forms its B fragment
                // (8 rows of its channel) in registers; the GS products take
                // dB's rows in lane groups 0, 1 and dP's in 2, 3 (transpose
                // reads), so one 16x16x32 step covers both terms of a block.
                // lane coordinates as opaque values: no address of this rare
                // branch is hoisted to where it would hold registers
                int l16 = ln, gq = g4, cx = ch, la_ = lane, bm = mi;
                asm volatile("" : "+v"(l16), "+v"(gq), "+v"(cx), "+v"(la_), "+v"(bm));
                auto rho_of = [&](int I) { return I == 0 ? 0.f : sm.gscan[4 * I * D + cx]; };
                const float rm = rho_of(bm);
                f32x4 aK = {0.f, 0.f, 0.f, 0.f}, aQ = aK;
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    if (32 * kc >= 16 * (bm + 1)) continue;
                    float yv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int s3 = 32 * kc + 8 * gq + j;
                        yv[j] = s3 < 16 * (bm + 1)
                                    ? bf16_to_f32(sm.kn[s3 * LDT + cx]) * gate_exp(rm - sm.g[s3 * LDG + cx])
                                    : 0.f;
                    }
                    const u32x4 yb = {pk(yv[0], yv[1]), pk(yv[2], yv[3]), pk(yv[4], yv[5]), pk(yv[6], yv[7])};
                    aK = mma32(frag<kKc>(dB + 16 * bm * LDC, LDC, 32 * kc, la_), yb, aK);
                    aQ = mma32(frag<kKc>(sm.dp + 16 * bm * LDC, LDC, 32 * kc, la_), yb, aQ);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float f = gate_exp(gr4[i] - rm);
                    fk[i] = aK[i] * f;
                    fq[i] = aQ[i] * f;
                }
                const bf16_t* asrc = gq < 2 ? dB : sm.dp;        // dB^T or dP^T rows
                const bf16_t* bsrc = gq < 2 ? sm.kn : sm.qg;     // k or q
#pragma unroll 1
                for (int I = bm; I < 4; ++I) {
                    const float rI = rho_of(I);
                    const int r0 = 16 * I + 8 * (gq & 1);
                    const bf16_t* pa = asrc + (r0 + (l16 >> 2)) * LDC + 16 * bm + 4 * (l16 & 3);
                    const u32x4 af = cat(ld_tr4(pa), ld_tr4(pa + 4 * LDC));
                    float xv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        xv[j] = bf16_to_f32(bsrc[(r0 + j) * LDT + cx]) *
                                gate_exp(sm.g[(r0 + j) * LDG + cx] - rI);
                    const u32x4 xb = {pk(xv[0], xv[1]), pk(xv[2], xv[3]), pk(xv[4], xv[5]), pk(xv[6], xv[7])};
                    const f32x4 a = mma32(af, xb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) gsum[i] += a[i] * gate_exp(rI - gr4[i]);
                }
            } else {
#pragma unroll 2
            for (int s2 = 0; s2 < C; ++s2) {
                const float ks = bf16_to_f32(sm.kn[s2 * LDT + ch]), qs = bf16_to_f32(sm.qg[s2 * LDT + ch]);
                const float gs = sm.g[s2 * LDG + ch];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mi + 4 * g4 + i;
                    // s2 as the column of row r, or as the row over row r
                    const float d = (gr4[i] - gs) * kLog2e;
                    const float e = __builtin_amdgcn_exp2f(s2 <= r ? d : -d);
                    if (s2 < r) fk[i] += bf16_to_f32(dB[r * LDC + s2]) * ks * e;
                    if (s2 <= r) fq[i] += bf16_to_f32(sm.dp[r * LDC + s2]) * ks * e;
                    if (s2 > r) gsum[i] += bf16_to_f32(dB[s2 * LDC + r]) * ks * e;
                    if (s2 >= r) gsum[i] += bf16_to_f32(sm.dp[s2 * LDC + r]) * qs * e;
                }
            }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mi + 4 * g4 + i;
                float dgv = 0.f;
                dkq[x][i] = 0u;
                if (r < c.len) {
                    const float eg = gate_exp(gr4[i]), ed = gate_exp(G - gr4[i]);
                    const float dKd = rKd[x][i];
                    const float kx = kv[x][i], qx = qv[x][i];
                    const float dkv = fk[i] + gsum[i] + rKgW[x][i] * eg + dKd * ed;
                    const float dqv = fq[i] + rQgS[x][i] * eg;
                    dkq[x][i] = uint32_t(bf(dkv)) | (uint32_t(bf(dqv)) << 16);
                    dgv = (fk[i] - gsum[i]) * kx + fq[i] * qx + rKgW[x][i] * kx * eg +
                          rQgS[x][i] * qx * eg - dKd * kx * ed;
                    dGp += dKd * kx * ed;
                }
                dgr[x][i] = dgv;
            }
        }
        // every wave has read the raw keys and queries: their buffers take dk and dq
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int mi = wave / 8 + 2 * x;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mi + 4 * g4 + i;
                if (r < c.len) {
                    sm.kg[r * LDT + ch] = uint16_t(dkq[x][i] & 0xffffu);   // dk
                    sm.kn[r * LDT + ch] = uint16_t(dkq[x][i] >> 16);       // dq
                }
            }
        }
    }
    __syncthreads();
    {
        const int r = tid / (D / 8), c8 = (tid % (D / 8)) * 8;
        if (r < c.len) {
            const int64_t row = ((c.t0 + r) * H + c.h) * D + c8;
            *reinterpret_cast<u32x4*>(dk + row) = *reinterpret_cast<const u32x4*>(sm.kg + r * LDT + c8);
            *reinterpret_cast<u32x4*>(dq + row) = *reinterpret_cast<const u32x4*>(sm.kn + r * LDT + c8);
        }
    }
    if constexpr (GATE != kGateNone) {
        // dlog_alpha[r] = sum_{r' >= r} dg[r'] + dG per key channel.  The row
        // blocks of a channel are split over waves cb and cb + 8: each
        // publishes its blocks' totals and its part of dG; then row r =
        // 16 mi + 4 g4 + i is summed over the rows after it in its lane (i),
        // in the lane groups after it (g4) and in the row blocks after it,
        // in that fixed order
        float tot[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const float s = (dgr[x][0] + dgr[x][1]) + (dgr[x][2] + dgr[x][3]);
            const float t2 = s + __shfl_xor(s, 16);
            tot[x] = t2 + __shfl_xor(t2, 32);
        }
        dGp += __shfl_xor(dGp, 16);
        dGp += __shfl_xor(dGp, 32);
        if (g4 == 0) {
            sm.ftot[wave / 8][ch] = tot[0];
            sm.ftot[wave / 8 + 2][ch] = tot[1];
            sm.fdg[wave / 8][ch] = dGp;
        }
        __syncthreads();
        const float dG = s_dgam[ch] * gate_exp(G) + (sm.fdg[0][ch] + sm.fdg[1][ch]);
        // per-channel gates: the results go straight into the gate buffer
        // (its last reads were before the barrier above) and leave in whole
        // 16-byte pieces of rows; per-head gates: kept for the channel sum
        float out[2][4];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int mi = wave / 8 + 2 * x;
            float after = dG;                     // rows of the row blocks after mi
            for (int m = 3; m > mi; --m) after += sm.ftot[m][ch];
            const float s = (dgr[x][0] + dgr[x][1]) + (dgr[x][2] + dgr[x][3]);
            const float s16 = __shfl_down(s, 16), s32 = __shfl_down(s, 32), s48 = __shfl_down(s, 48);
            const float groups_after = (g4 < 3 ? s16 : 0.f) + (g4 < 2 ? s32 : 0.f) +
                                       (g4 < 1 ? s48 : 0.f);
            float run = after + groups_after;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                run += dgr[x][i];
                if constexpr (GATE == kGateChannel) sm.g[(16 * mi + 4 * g4 + i) * LDG + ch] = run;
                else out[x][i] = run;
            }
        }
        if constexpr (GATE == kGateChannel) {
            __syncthreads();
#pragma unroll
            for (int x = 0; x < C * D / 4 / GG; ++x) {
                const int u = tid + GG * x, r = u / (D / 4), c4 = (u % (D / 4)) * 4;
                if (r < c.len)
                    *reinterpret_cast<f32x4*>(dla + ((c.t0 + r) * H + c.h) * D + c4) =
                        *reinterpret_cast<const f32x4*>(sm.g + r * LDG + c4);
            }
        } else {
            // one gate per (token, head) reaches every key channel: the sum
            // over the channels, per wave across its 16 lanes, then over the
            // channel blocks in order
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v2 = out[x][i];
#pragma unroll
                    for (int m = 1; m < 16; m <<= 1) v2 += __shfl_xor(v2, m);
                    if (ln == 0) sm.hp[cb][16 * (wave / 8 + 2 * x) + 4 * g4 + i] = v2;
                }
            __syncthreads();
            if (tid < C && tid < c.len) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < D / 16; ++w) acc += sm.hp[w][tid];
                dla[(c.t0 + tid) * H + c.h] = acc;
            }
        }
    }
}

// ===================================================================
// the fused input front-end around the backward: its activations ahead of
// the call (one 32-lane group per (token, head) row, 4 channels per lane,
// the forward front-end's arithmetic), and the chain rule through them
// after it, in place on the gradients:
//   x_n = x / n, n = max(||x||, eps):  dx = (dx_n - x_n (x_n . dx_n)) / n
//                                      (dx_n / eps below the floor)
//   log_alpha = -c softplus(g):        dg = -c sigmoid(g) dlog_alpha
//   beta = sigmoid(y):                 dy = beta (1 - beta) dbeta
// ===================================================================
constexpr int FT = 256;    // threads per block: 8 rows

__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

template <int GATE>
__global__ __launch_bounds__(FT)
void front_act_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, FrontEnd fe,
                      int64_t rows, bf16_t* __restrict__ qn, bf16_t* __restrict__ kn,
                      float* __restrict__ la, float* __restrict__ beta) {
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * FT + threadIdx.x) >> 5;
    const int j = threadIdx.x & 31;
    if (row >= rows) return;     // whole 32-lane groups leave together
    if (fe.l2norm) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16_t* x = (t == 0 ? q : k) + row * D + 4 * j;
            const u32x2 w = *reinterpret_cast<const u32x2*>(x);
            const float v[4] = {lo_bf(w[0]), hi_bf(w[0]), lo_bf(w[1]), hi_bf(w[1])};
            float s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) s2 += v[e] * v[e];
            const float inv = __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(group_sum(s2)), kFrontEps));
            *reinterpret_cast<u32x2*>((t == 0 ? qn : kn) + row * D + 4 * j) =
                u32x2{pk(v[0] * inv, v[1] * inv), pk(v[2] * inv, v[3] * inv)};
        }
    }
    if (fe.gate_pre) {
        if constexpr (GATE == kGateChannel) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(fe.gate_pre + row * D + 4 * j);
            const float x[4] = {lo_bf(w[0]), hi_bf(w[0]), lo_bf(w[1]), hi_bf(w[1])};
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = -fe.gate_scale * softplus_f32(x[e]);
            *reinterpret_cast<f32x4*>(la + row * D + 4 * j) = o;
        } else if (j == 0) {
            la[row] = -fe.gate_scale * softplus_f32(bf16_to_f32(fe.gate_pre[row]));
        }
    }
    if (fe.beta_pre && j == 0) beta[row] = sigmoid_f32(bf16_to_f32(fe.beta_pre[row]));
}

template <int GATE>
__global__ __launch_bounds__(FT)
void front_chain_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, FrontEnd fe,
                        int64_t rows, bf16_t* __restrict__ dq, bf16_t* __restrict__ dk,
                        float* __restrict__ dla, float* __restrict__ dbeta) {
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * FT + threadIdx.x) >> 5;
    const int j = threadIdx.x & 31;
    if (row >= rows) return;     // whole 32-lane groups leave together
    if (fe.l2norm) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x2 w = *reinterpret_cast<const u32x2*>((t == 0 ? q : k) + row * D + 4 * j);
            bf16_t* gp = (t == 0 ? dq : dk) + row * D + 4 * j;
            const u32x2 gw = *reinterpret_cast<const u32x2*>(gp);
            const float v[4] = {lo_bf(w[0]), hi_bf(w[0]), lo_bf(w[1]), hi_bf(w[1])};
            const float d[4] = {lo_bf(gw[0]), hi_bf(gw[0]), lo_bf(gw[1]), hi_bf(gw[1])};
            float s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) s2 += v[e] * v[e];
            const float nrm = __builtin_sqrtf(group_sum(s2));
            const float inv = __builtin_amdgcn_rcpf(fmaxf(nrm, kFrontEps));
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) p += v[e] * inv * d[e];
            p = group_sum(p);
            if (!(nrm > kFrontEps)) p = 0.f;            // below the floor n is constant
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (d[e] - v[e] * inv * p) * inv;
            *reinterpret_cast<u32x2*>(gp) = u32x2{pk(o[0], o[1]), pk(o[2], o[3])};
        }
    }
    if (fe.gate_pre) {
        if constexpr (GATE == kGateChannel) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(fe.gate_pre + row * D + 4 * j);
            const float x[4] = {lo_bf(w[0]), hi_bf(w[0]), lo_bf(w[1]), hi_bf(w[1])};
            f32x4 g = *reinterpret_cast<const f32x4*>(dla + row * D + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) g[e] *= -fe.gate_scale * sigmoid_f32(x[e]);
            *reinterpret_cast<f32x4*>(dla + row * D + 4 * j) = g;
        } else if (j == 0) {
            dla[row] *= -fe.gate_scale * sigmoid_f32(bf16_to_f32(fe.gate_pre[row]));
        }
    }
    if (fe.beta_pre && j == 0) {
        const float b = sigmoid_f32(bf16_to_f32(fe.beta_pre[row]));
        dbeta[row] *= b * (1.f - b);
    }
}

__global__ void bwd_init_kernel(const float* __restrict__ dhT, float* __restrict__ dstate,
                                int64_t n4) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n4;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (dhT) x = reinterpret_cast<const f32x4*>(dhT)[i];
        reinterpret_cast<f32x4*>(dstate)[i] = x;
    }
}

int64_t bound_chunks(int64_t total_T) { return total_T > 0 ? (total_T + C - 1) / C : 0; }

// Per-block buffers come in pairs: while the gradient pass of block b reads
// its pair, the prep and the carry of block b - 1 fill the other.
constexpr int kRing = 3;

struct BwdLayout {
    size_t fwd, sall, slots, dsblk, deblk, dstate, total;
};

// have_states: the chunk states come from the caller (no forward pass, no
// record in the workspace)
BwdLayout bwd_layout(int64_t total_T, int32_t N, int32_t H, int L_b, bool have_states) {
    BwdLayout l;
    const size_t nh = static_cast<size_t>(N) * H;
    const size_t blk = nh * L_b;
    l.fwd = have_states ? 0 : wy_workspace_bytes(N, H, D, D, wy_default_block_chunks(total_T, N, H, D));
    l.sall = have_states ? 0
                         : (static_cast<size_t>(N) + static_cast<size_t>(bound_chunks(total_T)) + 1) *
                               H * kState * 2;
    l.slots = blk * kSlot;
    l.dsblk = blk * kState * 2;
    l.deblk = blk * C * D * 2;
    l.dstate = nh * kState * 4;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    l.total = up(l.fwd) + up(l.sall) + kRing * (up(l.slots) + up(l.dsblk) + up(l.deblk)) +
              up(l.dstate);
    return l;
}

// the device of the caller's stream is current for the call (the second
// stream and the events must live on it); the previous device is restored
struct DeviceOfStream {
    int prev = -1;
    hipError_t set(hipStream_t stream) {
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess || !stream) return e;
        int dev = prev;
        if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
        return dev == prev ? hipSuccess : hipSetDevice(dev);
    }
    ~DeviceOfStream() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// events of one call, released when the call returns (a destroyed event
// still completes the waits already queued on it)
struct CallEvents {
    hipEvent_t start = nullptr, grad[kRing] = {}, carry[kRing] = {};
    hipError_t create() {
        hipError_t e = hipEventCreateWithFlags(&start, hipEventDisableTiming);
        for (int i = 0; i < kRing && e == hipSuccess; ++i) {
            e = hipEventCreateWithFlags(&grad[i], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&carry[i], hipEventDisableTiming);
        }
        return e;
    }
    ~CallEvents() {
        if (start) (void)hipEventDestroy(start);
        for (int i = 0; i < kRing; ++i) {
            if (grad[i]) (void)hipEventDestroy(grad[i]);
            if (carry[i]) (void)hipEventDestroy(carry[i]);
        }
    }
};

}  // namespace

int bwd_default_block_chunks(int64_t seq_bound, int32_t N, int32_t H) {
    // about 1.25 GiB of per-block buffers (prep operands and carry outputs:
    // ~155 KB per (chunk, head), three blocks' worth), at most 80 chunks
    // (measured at 32 heads: 64, 72, 80 and 88 chunks per block)
    const size_t per_chunk = static_cast<size_t>(N) * H * kRing *
                             (kSlot + kState * 2 + static_cast<size_t>(C) * D * 2);
    int64_t L = static_cast<int64_t>((size_t{5} << 28) / per_chunk);
    L = std::max<int64_t>(1, std::min<int64_t>(L, std::max<int64_t>(1, bound_chunks(seq_bound))));
    return static_cast<int>(std::min<int64_t>(L, 80));
}

// the front-end's activated inputs: normalised q and k (bf16), log_alpha
// and beta (fp32), each present when its part of the front-end is on
struct FrontLayout {
    size_t qk, la, beta, total;
};
FrontLayout front_layout(int64_t total_T, int32_t H, int gate, const FrontEnd& fe) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = static_cast<size_t>(total_T) * H;
    FrontLayout f;
    f.qk = fe.l2norm ? rows * D * 2 : 0;
    f.la = fe.gate_pre ? rows * (gate == kGateChannel ? D : 1) * 4 : 0;
    f.beta = fe.beta_pre ? rows * 4 : 0;
    f.total = 2 * up(f.qk) + up(f.la) + up(f.beta);
    return f;
}

size_t bwd_workspace_bytes(int64_t total_T, int32_t N, int32_t H, int L_b, int gate,
                           const FrontEnd& fe, bool have_states) {
    return (fe.active() ? front_layout(total_T, H, gate, fe).total : 0) +
           bwd_layout(total_T, N, H, L_b, have_states).total;
}

hipError_t launch_backward_core(const BackwardArgs& a, int L_b, void* ws, hipStream_t stream);

hipError_t launch_backward(const BackwardArgs& a, int L_b, void* ws, hipStream_t stream) {
    if (!a.fe.active()) return launch_backward_core(a, L_b, ws, stream);
    // activations ahead, the recurrence's backward on them, the chain rule after
    const FrontLayout f = front_layout(a.total_T, a.H, a.gate, a.fe);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    uint8_t* p = static_cast<uint8_t*>(ws);
    bf16_t* qn = reinterpret_cast<bf16_t*>(p);         p += up(f.qk);
    bf16_t* kn = reinterpret_cast<bf16_t*>(p);         p += up(f.qk);
    float* la = reinterpret_cast<float*>(p);           p += up(f.la);
    float* be = reinterpret_cast<float*>(p);           p += up(f.beta);
    BackwardArgs b = a;
    b.fe = FrontEnd{};
    if (a.fe.l2norm) { b.q = qn; b.k = kn; }
    if (a.fe.gate_pre) b.log_alpha = la;
    if (a.fe.beta_pre) b.beta = be;
    const int64_t rows = a.total_T * a.H;
    const unsigned blocks = static_cast<unsigned>((rows * 32 + FT - 1) / FT);
    const bf16_t* q = static_cast<const bf16_t*>(a.q);
    const bf16_t* k = static_cast<const bf16_t*>(a.k);
    hipError_t e;
    if (rows > 0) {
        auto act = a.gate == kGateChannel ? front_act_kernel<kGateChannel> : front_act_kernel<kGateHead>;
        hipLaunchKernelGGL(act, dim3(blocks), dim3(FT), 0, stream, q, k, a.fe, rows, qn, kn, la, be);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_backward_core(b, L_b, p, stream)) != hipSuccess) return e;
    if (rows > 0) {
        auto chain = a.gate == kGateChannel ? front_chain_kernel<kGateChannel>
                                            : front_chain_kernel<kGateHead>;
        hipLaunchKernelGGL(chain, dim3(blocks), dim3(FT), 0, stream, q, k, a.fe, rows,
                           static_cast<bf16_t*>(a.dq), static_cast<bf16_t*>(a.dk), a.dlog_alpha,
                           a.dbeta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_backward_core(const BackwardArgs& a, int L_b, void* ws, hipStream_t stream) {
    const BwdLayout l = bwd_layout(a.total_T, a.N, a.H, L_b, a.states != nullptr);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    uint8_t* p = static_cast<uint8_t*>(ws);
    uint8_t* fwd_ws = p;          p += up(l.fwd);
    const bf16_t* sall = a.states ? static_cast<const bf16_t*>(a.states)
                                  : reinterpret_cast<bf16_t*>(p);
    p += up(l.sall);
    uint8_t* slots[kRing];
    bf16_t* dsblk[kRing];
    bf16_t* deblk[kRing];
    for (int i = 0; i < kRing; ++i) {
        slots[i] = p;                                  p += up(l.slots);
        dsblk[i] = reinterpret_cast<bf16_t*>(p);       p += up(l.dsblk);
        deblk[i] = reinterpret_cast<bf16_t*>(p);       p += up(l.deblk);
    }
    float* dstate = reinterpret_cast<float*>(p);
    // with a second stream, the events that order it against the caller's
    // are created on the device of the streams (the previous device is
    // restored); without one, everything runs in order on the caller's
    // stream and no event is needed
    const bool two = a.aux != nullptr;
    hipStream_t serial = two ? a.aux : stream;
    DeviceOfStream on_device;
    CallEvents ev;
    hipError_t e = hipSuccess;
    if (two) {
        if ((e = on_device.set(stream)) != hipSuccess) return e;
        if ((e = ev.create()) != hipSuccess) return e;
    }

    // 1. forward: the state after every full chunk, no outputs (unless the
    //    caller passes the record of its own forward pass)
    if (!a.states) {
        PrefillArgs f{};
        f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.beta = a.beta; f.h0 = a.h0;
        f.cu_seqlens = a.cu_seqlens; f.o = nullptr; f.hT = nullptr; f.order = nullptr;
        f.total_T = a.total_T; f.N = a.N; f.H = a.H; f.d_k = D; f.d_v = D; f.gate = a.gate;
        f.dtype_f32 = false; f.scale = a.scale;
        f.snapshots = reinterpret_cast<float*>(const_cast<bf16_t*>(sall));   // bf16 record (snap_cap < 0)
        f.snap_tokens = C; f.snap_cap = -1;
        f.max_seqlen = a.max_seqlen;
        e = launch_prefill_wy(f, D / 16, wy_default_block_chunks(a.seq_bound(), a.N, a.H, D), fwd_ws,
                              stream);
        if (e != hipSuccess) return e;
    }

    // 2. backward over blocks of chunks, from the last.  Second stream:
    //    prep(b), then carry(b); caller's stream: grad(b) once carry(b) is
    //    done, so grad(b) runs beside prep(b - 1) and carry(b - 1).  Ring
    //    slot b % 3 holds block b's operands and carry outputs; prep(b)
    //    reuses the slot of block b + 3 and first waits for its last
    //    reader, grad(b + 3).  The second stream starts after the caller's
    //    earlier work, and the caller's stream ends with grad(0), which
    //    waits for the last carry: the call's work is whole on the caller's
    //    stream.
    const int64_t n4 = static_cast<int64_t>(a.N) * a.H * kState / 4;
    hipLaunchKernelGGL(bwd_init_kernel, dim3(static_cast<unsigned>(std::min<int64_t>(4096, (n4 + 255) / 256))),
                       dim3(256), 0, stream, a.dhT, dstate, n4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t bound = std::max<int64_t>(1, bound_chunks(a.seq_bound()));
    const int64_t nblk = (bound + L_b - 1) / L_b;
    const unsigned chunks = static_cast<unsigned>(static_cast<int64_t>(a.N) * L_b * a.H);
    const bf16_t* q = static_cast<const bf16_t*>(a.q);
    const bf16_t* k = static_cast<const bf16_t*>(a.k);
    const bf16_t* v = static_cast<const bf16_t*>(a.v);
    const bf16_t* dO = static_cast<const bf16_t*>(a.dO);
    auto prep = a.gate == kGateChannel ? bwd_prep_kernel<kGateChannel>
              : a.gate == kGateHead    ? bwd_prep_kernel<kGateHead>
                                       : bwd_prep_kernel<kGateNone>;
    auto gk = a.gate == kGateChannel ? bwd_grad_kernel<bf16_t, kGateChannel>
            : a.gate == kGateHead    ? bwd_grad_kernel<bf16_t, kGateHead>
                                     : bwd_grad_kernel<bf16_t, kGateNone>;
    if (two) {
        if ((e = hipEventRecord(ev.start, stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(serial, ev.start, 0)) != hipSuccess) return e;
    }
    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int c_lo = static_cast<int>(b * L_b), r = static_cast<int>(b % kRing);
        if (two && b + kRing < nblk && (e = hipStreamWaitEvent(serial, ev.grad[r], 0)) != hipSuccess)
            return e;
        if (a.total_T > 0) {    // nothing to prepare for an empty batch
            hipLaunchKernelGGL(prep, dim3(chunks), dim3(GT), 0, serial, q, k, a.log_alpha,
                               a.beta, a.cu_seqlens, a.H, c_lo, L_b, a.scale, slots[r]);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL(bwd_carry_kernel, dim3(static_cast<unsigned>(a.N * a.H * (D / kCarryTile))),
                           dim3(GG), 0, serial, slots[r], dO, a.cu_seqlens, a.N, a.H, c_lo, L_b,
                           static_cast<int>(bound), dstate, dsblk[r], deblk[r], a.dh0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (two) {
            if ((e = hipEventRecord(ev.carry[r], serial)) != hipSuccess) return e;
            if ((e = hipStreamWaitEvent(stream, ev.carry[r], 0)) != hipSuccess) return e;
        }
        if (a.total_T == 0) continue;
        hipLaunchKernelGGL(gk, dim3(chunks), dim3(GG), 0, stream, slots[r], dsblk[r], deblk[r],
                           sall, a.h0, q, k, v, dO, a.log_alpha, a.beta, a.cu_seqlens, a.H, c_lo,
                           L_b, a.scale, static_cast<bf16_t*>(a.dq), static_cast<bf16_t*>(a.dk),
                           static_cast<bf16_t*>(a.dv), a.dlog_alpha, a.dbeta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (two && (e = hipEventRecord(ev.grad[r], stream)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
