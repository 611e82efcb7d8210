// kda_exact.h -- the exact pairwise form of a chunk's decay-weighted
// products, for chunks whose cumulative gate leaves the range of the
// factored form e^{g} e^{-g} (there e^{-g} overflows fp32, although every
// factor the products need lies in (0, 1]):
//   Araw[r][s] = sum_c k_r[c] k_s[c] e^{g_r[c] - g_s[c]}        (s <= r)
//   P[r][s]    = sum_c q_r[c] k_s[c] e^{g_r[c] - g_s[c]}
// with every factor formed from a difference of cumulative gates.  The
// rows of k, q and g are staged through LDS 32 key channels at a time
// (rows of XS floats); 512 threads share the 2080 entries with s <= r:
//   threads 0..479:   the 240 blocks of 4 rows x 2 columns strictly below
//                     the diagonal 4x4 blocks, two threads each, 16 of
//                     every 32 staged channels apiece (adjacent lanes);
//   threads 480..511: the 32 blocks of 4 x 2 that make up the diagonal 4x4
//                     blocks, one thread each, all 32 staged channels.
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kExactXS = 33;      // fp32 stride of a staged row of 32 channels
constexpr int kExactThreads = 512;

struct ExactUnit {
    int bi, bj;       // rows 4 bi .. +3, columns 2 bj .. +1
    int c0, cw;       // staged channels c0 .. c0 + cw - 1 of each round
    bool diag;        // one of the diagonal 4x4 blocks' halves
};

__device__ __forceinline__ ExactUnit exact_unit(int tid) {
    ExactUnit u;
    u.diag = tid >= 480;
    if (!u.diag) {
        const int b = tid >> 1;          // row block bi holds 2 bi column pairs
        int bi = static_cast<int>((1.f + __builtin_sqrtf(1.f + 4.f * static_cast<float>(b))) * 0.5f);
        while (bi * (bi - 1) > b) --bi;
        while ((bi + 1) * bi <= b) ++bi;
        u.bi = bi;
        u.bj = b - bi * (bi - 1);
        u.cw = 16;
        u.c0 = 16 * (tid & 1);
    } else {
        const int d = tid - 480;
        u.bi = d >> 1;
        u.bj = 2 * u.bi + (d & 1);
        u.cw = 32;
        u.c0 = 0;
    }
    return u;
}

// Adds one round's staged channels to this unit's entries.  gscale turns a
// gate difference into the argument of exp2 (1 for gates in log2 units,
// log2(e) for natural ones).
__device__ __forceinline__ void exact_accumulate(const ExactUnit& u, const float* sk,
                                                 const float* sq, const float* sg, float gscale,
                                                 float (&a)[4][2], float (&p)[4][2]) {
#pragma unroll 1
    for (int cc = 0; cc < u.cw; ++cc) {
        const int c = u.c0 + cc;
        float kr[4], qr[4], gr[4], ks[2], gs[2];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            kr[x] = sk[(4 * u.bi + x) * kExactXS + c];
            qr[x] = sq[(4 * u.bi + x) * kExactXS + c];
            gr[x] = sg[(4 * u.bi + x) * kExactXS + c];
        }
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            ks[y] = sk[(2 * u.bj + y) * kExactXS + c];
            gs[y] = sg[(2 * u.bj + y) * kExactXS + c];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                if (2 * u.bj + y > 4 * u.bi + x) continue;   // above the diagonal
                const float w = ks[y] * __builtin_amdgcn_exp2f((gr[x] - gs[y]) * gscale);
                a[x][y] = __builtin_fmaf(kr[x], w, a[x][y]);
                p[x][y] = __builtin_fmaf(qr[x], w, p[x][y]);
            }
    }
}

// Sums the two channel halves of an off-diagonal block (adjacent lanes).
__device__ __forceinline__ void exact_reduce(const ExactUnit& u, float (&a)[4][2], float (&p)[4][2]) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const float ta = a[x][y] + __shfl_xor(a[x][y], 1);
            const float tp = p[x][y] + __shfl_xor(p[x][y], 1);
            a[x][y] = u.diag ? a[x][y] : ta;
            p[x][y] = u.diag ? p[x][y] : tp;
        }
}

// whether this thread writes its unit's entries (one thread per unit)
__device__ __forceinline__ bool exact_writer(const ExactUnit& u, int tid) {
    return u.diag || (tid & 1) == 0;
}

}  // namespace kda
