// kda_api.cpp -- the C entry points declared in include/kda.h.
//
// Each entry point validates every argument on the host (null pointers,
// sizes and their byte-count overflow, supported head dimensions and dtype,
// 16-byte alignment, aliasing of outputs with inputs, workspace size) and
// only then enqueues kernels on the caller's stream.  Nothing here
// allocates, synchronises or keeps state between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

constexpr int kAbiVersion = 12;
// the automatic choice takes the two-pass matrix path below this many
// (sequence, head) pairs: there the fused kernel would split each pair into
// 4 or more value tiles that all redo the pair's state-independent work
constexpr int64_t kTwoPassMaxPairs = 128;
constexpr size_t kWorkspaceAlign = 256;

bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// a * b without signed overflow, for non-negative operands.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Common size validation; fills byte counts.  Returns a kda_status.
struct Sizes {
    int64_t qk_bytes, v_bytes, la_bytes, beta_bytes, state_bytes;
};

int check_sizes(int64_t tokens, int64_t N, int64_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                int32_t gate, Sizes* sz) {
    if (N < 1 || H < 1 || tokens < 0) return KDA_STATUS_INVALID_ARGUMENT;
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_NONE)
        return KDA_STATUS_INVALID_ARGUMENT;
    if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_F32) return KDA_STATUS_UNSUPPORTED;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_STATUS_UNSUPPORTED;
    const int64_t esz = dtype == KDA_DTYPE_F32 ? 4 : 2;
    int64_t th, x;
    if (!mul_ok(tokens, H, &th)) return KDA_STATUS_INVALID_ARGUMENT;
    if (!mul_ok(th, d_k, &x) || !mul_ok(x, 4, &sz->la_bytes)) return KDA_STATUS_INVALID_ARGUMENT;
    if (gate == KDA_GATE_HEAD) sz->la_bytes = th * 4;
    if (gate == KDA_GATE_NONE) sz->la_bytes = 0;
    if (!mul_ok(th, d_k, &x) || !mul_ok(x, esz, &sz->qk_bytes)) return KDA_STATUS_INVALID_ARGUMENT;
    if (!mul_ok(th, d_v, &x) || !mul_ok(x, esz, &sz->v_bytes)) return KDA_STATUS_INVALID_ARGUMENT;
    if (!mul_ok(th, 4, &sz->beta_bytes)) return KDA_STATUS_INVALID_ARGUMENT;
    int64_t nh;
    if (!mul_ok(N, H, &nh) || !mul_ok(nh, d_k, &x) || !mul_ok(x, d_v, &x) ||
        !mul_ok(x, 4, &sz->state_bytes))
        return KDA_STATUS_INVALID_ARGUMENT;
    // keep every byte count (and the largest launch grid) far from int64 and
    // 32-bit grid limits: 2^31 work-groups at most, 2^62 bytes at most
    if (nh > (int64_t{1} << 27)) return KDA_STATUS_INVALID_ARGUMENT;
    if (!mul_ok(th, d_k, &x) || !mul_ok(x, 4, &x) || x > (int64_t{1} << 62))
        return KDA_STATUS_INVALID_ARGUMENT;
    if (sz->state_bytes > (int64_t{1} << 62))
        return KDA_STATUS_INVALID_ARGUMENT;
    return KDA_STATUS_OK;
}

// log_alpha is required unless the call has no gate; a per-channel gate is
// vector-loaded (16 bytes), a per-head gate read as scalars (4 bytes)
int check_gate_ptr(int32_t gate, const float* log_alpha, bool needed) {
    if (gate == KDA_GATE_NONE || !needed) return KDA_STATUS_OK;
    if (!log_alpha) return KDA_STATUS_INVALID_ARGUMENT;
    if (gate == KDA_GATE_CHANNEL ? !aligned16(log_alpha) : !aligned4(log_alpha))
        return KDA_STATUS_MISALIGNED;
    return KDA_STATUS_OK;
}

// The fused input front-end: checks and conversion.  With gate_pre the
// caller's log_alpha must be NULL (and a gate layout other than none); with
// beta_pre the caller's beta must be NULL.  *la_needed / *beta_needed tell
// the caller whether log_alpha / beta are still required.
int check_front(const kda_front_end* f, int32_t gate, const float* log_alpha, const float* beta,
                int64_t tokens, int64_t H, int32_t d_k, kda::FrontEnd* fe, bool* la_needed,
                bool* beta_needed, Range* r_gate, Range* r_beta) {
    *fe = kda::FrontEnd{};
    *la_needed = true;
    *beta_needed = true;
    *r_gate = Range{0, 0};
    *r_beta = Range{0, 0};
    if (!f) return KDA_STATUS_OK;
    fe->l2norm = f->l2norm_qk != 0;
    if (f->gate_pre) {
        if (gate == KDA_GATE_NONE || log_alpha) return KDA_STATUS_INVALID_ARGUMENT;
        if (!std::isfinite(f->gate_scale) || f->gate_scale < 0.f) return KDA_STATUS_INVALID_ARGUMENT;
        if (gate == KDA_GATE_CHANNEL ? !aligned16(f->gate_pre)
                                     : (reinterpret_cast<uintptr_t>(f->gate_pre) & 1u))
            return KDA_STATUS_MISALIGNED;
        fe->gate_pre = static_cast<const uint16_t*>(f->gate_pre);
        fe->gate_scale = f->gate_scale;
        *la_needed = false;
        *r_gate = range_of(f->gate_pre, tokens * H * (gate == KDA_GATE_CHANNEL ? d_k : 1) * 2);
    }
    if (f->beta_pre) {
        if (beta) return KDA_STATUS_INVALID_ARGUMENT;
        if (reinterpret_cast<uintptr_t>(f->beta_pre) & 1u) return KDA_STATUS_MISALIGNED;
        fe->beta_pre = static_cast<const uint16_t*>(f->beta_pre);
        *beta_needed = false;
        *r_beta = range_of(f->beta_pre, tokens * H * 2);
    }
    return KDA_STATUS_OK;
}

size_t plan_bytes(int32_t N) { return round_up(static_cast<size_t>(N) * sizeof(int32_t), kWorkspaceAlign); }

// Sizes-only view of a prefill for the path checks.
kda::PrefillArgs shape_args(int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                            int32_t dtype) {
    kda::PrefillArgs a{};
    a.total_T = total_T; a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.dtype_f32 = dtype == KDA_DTYPE_F32;
    return a;
}

// The kernel path, its tiling and the workspace it needs.
struct Plan {
    int32_t path;      // VECTOR, MATRIX or MATRIX_TWO_PASS
    int R;             // value tiles (matrix paths)
    int L_b;           // chunks per block (two-pass)
    size_t ws_bytes;   // scheduling table [+ two-pass slots and state copy]
};

// Sizes must already have passed check_sizes.
// budget > 0: the automatic two-pass block length is capped so that the
// workspace fits in budget bytes (the allocation-free entry point)
int resolve(int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
            const kda_prefill_options* options, Plan* pl, size_t budget = 0) {
    const int32_t path = options ? options->path : KDA_PATH_AUTO;
    const int32_t tiles = options ? options->value_tiles : 0;
    const int32_t blk = options ? options->block_chunks : 0;
    if (path < KDA_PATH_AUTO || path > KDA_PATH_MATRIX_TWO_PASS) return KDA_STATUS_INVALID_ARGUMENT;
    if (tiles < 0 || blk < 0) return KDA_STATUS_INVALID_ARGUMENT;
    if (options && options->max_seqlen < 0) return KDA_STATUS_INVALID_ARGUMENT;
    kda::PrefillArgs a = shape_args(total_T, N, H, d_k, d_v, dtype);
    a.max_seqlen = options ? options->max_seqlen : 0;
    const bool matrix_ok = kda::mfma_supported(a) && kda::wy_supported(a);
    if ((path == KDA_PATH_MATRIX || path == KDA_PATH_MATRIX_TWO_PASS) && !matrix_ok)
        return KDA_STATUS_UNSUPPORTED;
    // the per-chunk state record is written by the two-pass carry (bf16, d = 128)
    const bool record = options && options->chunk_states;
    if (record && (path == KDA_PATH_VECTOR || path == KDA_PATH_MATRIX || !matrix_ok ||
                   d_k != 128 || d_v != 128 || dtype != KDA_DTYPE_BF16))
        return KDA_STATUS_UNSUPPORTED;
    pl->path = path;
    if (path == KDA_PATH_AUTO) {
        pl->path = !matrix_ok ? KDA_PATH_VECTOR
                   : record || static_cast<int64_t>(N) * H < kTwoPassMaxPairs
                       ? KDA_PATH_MATRIX_TWO_PASS
                       : KDA_PATH_MATRIX;
    }
    pl->R = 0;
    pl->L_b = 0;
    pl->ws_bytes = plan_bytes(N);
    if (pl->path == KDA_PATH_VECTOR) return KDA_STATUS_OK;
    const bool two = pl->path == KDA_PATH_MATRIX_TWO_PASS;
    if (tiles > 0 && !(two ? kda::wy_tiles_ok(d_v, tiles) : kda::mfma_tiles_ok(d_v, tiles)))
        return KDA_STATUS_INVALID_ARGUMENT;
    pl->R = tiles > 0 ? tiles : two ? kda::wy_value_tiles(a) : kda::mfma_value_tiles(a);
    if (two) {
        pl->L_b = blk > 0 ? blk : kda::wy_default_block_chunks(a.seq_bound(), N, H, d_v);
        if (blk == 0 && budget > 0) {
            // the largest block length whose workspace fits the budget
            const size_t fixed = plan_bytes(N) + kda::wy_workspace_bytes(N, H, d_k, d_v, 0);
            const size_t per = kda::wy_workspace_bytes(N, H, d_k, d_v, 1) -
                               kda::wy_workspace_bytes(N, H, d_k, d_v, 0);
            const size_t fit = budget > fixed + kWorkspaceAlign
                                   ? (budget - fixed - kWorkspaceAlign) / per : 0;
            pl->L_b = static_cast<int>(std::max<size_t>(1, std::min<size_t>(pl->L_b, fit)));
        }
        if (!kda::wy_block_chunks_ok(N, H, pl->L_b)) return KDA_STATUS_INVALID_ARGUMENT;
        pl->ws_bytes += kda::wy_workspace_bytes(N, H, d_k, d_v, pl->L_b);
    }
    return KDA_STATUS_OK;
}

// bytes of the per-chunk state record: one bf16 state per (chunk index,
// head) over N + ceil(total_T / 64) + 1 indices (0 on overflow)
int64_t chunk_states_bytes(int64_t total_T, int32_t N, int32_t H) {
    const int64_t idx = static_cast<int64_t>(N) + (total_T + 63) / 64 + 1;
    int64_t bytes;
    if (!mul_ok(idx * H, int64_t{128} * 128 * 2, &bytes) || bytes > (int64_t{1} << 62)) return 0;
    return bytes;
}

// the shapes the backward (and the chunk-state record it reads) supports:
// the two-pass kernels' head bound (their 32-bit in-kernel offsets)
bool bwd_shape_ok(int32_t N, int32_t H) {
    return kda::wy_supported(shape_args(0, N, H, 128, 128, KDA_DTYPE_BF16));
}

// ---- the allocation-free prefill: its workspace is this array
// Each GPU the library runs on holds one copy of it until the process ends.
// In host code its name is only a stand-in for the symbol: every use of the
// memory goes through the device address looked up below.
constexpr size_t kNoAllocBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of the array on the device of `stream`, looked up
// once per device with that device current (the previous device is
// restored) and kept.
int scratch_of(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return KDA_STATUS_HIP_ERROR;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess) return KDA_STATUS_HIP_ERROR;
        if (prev != dev && hipSetDevice(dev) != hipSuccess) return KDA_STATUS_HIP_ERROR;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (prev != dev) (void)hipSetDevice(prev);
        if (e != hipSuccess || !ptr) return KDA_STATUS_HIP_ERROR;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return KDA_STATUS_OK;
}

int prefill_call(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* h0, const int32_t* cu_seqlens, int64_t total_T,
                 int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, float scale,
                 void* o, float* hT, void* workspace, size_t workspace_bytes,
                 const kda_prefill_options* options, void* stream, bool use_scratch);

}  // namespace

extern "C" {

int kda_abi_version(void) { return kAbiVersion; }

size_t kda_chunk_states_bytes(int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v) {
    Sizes sz;
    if (check_sizes(total_T, N, H, d_k, d_v, KDA_DTYPE_BF16, KDA_GATE_CHANNEL, &sz) !=
        KDA_STATUS_OK)
        return 0;
    if (d_k != 128 || d_v != 128 || !bwd_shape_ok(N, H)) return 0;
    return static_cast<size_t>(chunk_states_bytes(total_T, N, H));
}

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_STATUS_OK: return "ok";
        case KDA_STATUS_INVALID_ARGUMENT: return "invalid argument";
        case KDA_STATUS_UNSUPPORTED: return "unsupported head dimension or dtype";
        case KDA_STATUS_MISALIGNED: return "pointer misaligned (16 bytes; beta and cu_seqlens 4)";
        case KDA_STATUS_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_STATUS_HIP_ERROR: return "HIP kernel launch failed";
    }
    return "unknown status";
}

size_t kda_fwd_prefill_workspace_bytes_ex(int64_t total_T, int32_t N, int32_t H, int32_t d_k,
                                          int32_t d_v, int32_t dtype,
                                          const kda_prefill_options* options) {
    Sizes sz;
    if (check_sizes(total_T, N, H, d_k, d_v, dtype, options ? options->gate : 0, &sz) !=
        KDA_STATUS_OK)
        return 0;
    Plan pl;
    if (resolve(total_T, N, H, d_k, d_v, dtype, options, &pl) != KDA_STATUS_OK) return 0;
    return pl.ws_bytes;
}

size_t kda_fwd_prefill_workspace_bytes(int64_t total_T, int32_t N, int32_t H, int32_t d_k,
                                       int32_t d_v, int32_t dtype) {
    return kda_fwd_prefill_workspace_bytes_ex(total_T, N, H, d_k, d_v, dtype, nullptr);
}

int kda_fwd_prefill_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                       int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                       int32_t dtype, float scale, void* o, float* hT, void* workspace,
                       size_t workspace_bytes, const kda_prefill_options* options,
                       void* stream) {
    return prefill_call(q, k, v, log_alpha, beta, h0, cu_seqlens, total_T, N, H, d_k, d_v, dtype,
                        scale, o, hT, workspace, workspace_bytes, options, stream, false);
}

int kda_fwd_prefill_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                            const float* beta, const float* h0, const int32_t* cu_seqlens,
                            int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                            int32_t dtype, float scale, void* o, float* hT,
                            const kda_prefill_options* options, void* stream) {
    return prefill_call(q, k, v, log_alpha, beta, h0, cu_seqlens, total_T, N, H, d_k, d_v, dtype,
                        scale, o, hT, nullptr, 0, options, stream, true);
}

}  // extern "C"

namespace {
// kda_fwd_prefill_ex, or with use_scratch the allocation-free variant: every
// host check first, then (only then) the device array's address
int prefill_call(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* h0, const int32_t* cu_seqlens, int64_t total_T,
                 int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, float scale,
                 void* o, float* hT, void* workspace, size_t workspace_bytes,
                 const kda_prefill_options* options, void* stream, bool use_scratch) {
    const int32_t gate = options ? options->gate : KDA_GATE_CHANNEL;
    Sizes sz;
    const int st = check_sizes(total_T, N, H, d_k, d_v, dtype, gate, &sz);
    if (st != KDA_STATUS_OK) return st;
    if (!std::isfinite(scale)) return KDA_STATUS_INVALID_ARGUMENT;
    if (!cu_seqlens) return KDA_STATUS_INVALID_ARGUMENT;
    kda::FrontEnd fe;
    bool la_needed, beta_needed;
    Range r_gp, r_bp;
    const int fs = check_front(options ? &options->front : nullptr, gate, log_alpha, beta,
                               total_T, H, d_k, &fe, &la_needed, &beta_needed, &r_gp, &r_bp);
    if (fs != KDA_STATUS_OK) return fs;
    if (total_T > 0 && (!q || !k || !v || (beta_needed && !beta) || !o))
        return KDA_STATUS_INVALID_ARGUMENT;
    const int gs = check_gate_ptr(gate, log_alpha, total_T > 0 && la_needed);
    if (gs != KDA_STATUS_OK) return gs;
    if (gate == KDA_GATE_NONE) log_alpha = nullptr;   // never read
    // vector-loaded tensors need 16 bytes; beta and cu_seqlens are read as scalars
    const void* ptrs[] = {q, k, v, h0, o, hT, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_STATUS_MISALIGNED;
    if (!aligned4(beta) || !aligned4(cu_seqlens)) return KDA_STATUS_MISALIGNED;
    Plan pl;
    const int rs = resolve(total_T, N, H, d_k, d_v, dtype, options, &pl,
                           use_scratch ? kNoAllocBytes : 0);
    if (rs != KDA_STATUS_OK) return rs;
    const size_t need = pl.ws_bytes;
    if (use_scratch) {
        if (need > kNoAllocBytes) return KDA_STATUS_WORKSPACE_TOO_SMALL;   // beyond the array
    } else if (workspace_bytes < need || (need > 0 && !workspace)) {
        return KDA_STATUS_WORKSPACE_TOO_SMALL;
    }

    // outputs may not overlap inputs (hT == h0 exactly is allowed)
    const Range r_o = range_of(o, sz.v_bytes);
    const Range r_hT = range_of(hT, hT ? sz.state_bytes : 0);
    const Range r_ws = range_of(workspace, static_cast<int64_t>(need));
    const Range inputs[] = {range_of(q, sz.qk_bytes),       range_of(k, sz.qk_bytes),
                            range_of(v, sz.v_bytes),        range_of(log_alpha, sz.la_bytes),
                            range_of(beta, sz.beta_bytes),  range_of(cu_seqlens, (N + 1) * 4),
                            range_of(h0, h0 ? sz.state_bytes : 0)};
    for (const Range& in : inputs) {
        if (overlaps(r_o, in) || overlaps(r_ws, in)) return KDA_STATUS_INVALID_ARGUMENT;
    }
    for (const Range& in : {r_gp, r_bp}) {
        if (overlaps(r_o, in) || overlaps(r_ws, in) || overlaps(r_hT, in))
            return KDA_STATUS_INVALID_ARGUMENT;
    }
    for (int i = 0; i < 6; ++i)
        if (overlaps(r_hT, inputs[i])) return KDA_STATUS_INVALID_ARGUMENT;
    if (h0 && hT && h0 != hT && overlaps(r_hT, inputs[6])) return KDA_STATUS_INVALID_ARGUMENT;
    if (overlaps(r_o, r_hT) || overlaps(r_o, r_ws) || overlaps(r_hT, r_ws))
        return KDA_STATUS_INVALID_ARGUMENT;

    // state snapshots: [N][capacity][H][d_k][d_v] fp32, overlapping nothing
    const int32_t snap = options ? options->snapshot_tokens : 0;
    float* snaps = nullptr;
    int32_t cap = 0;
    if (snap != 0) {
        cap = options->snapshot_capacity;
        snaps = options->snapshots;
        if (snap < 0 || snap % 64 != 0 || cap < 1 || !snaps) return KDA_STATUS_INVALID_ARGUMENT;
        if (!aligned16(snaps)) return KDA_STATUS_MISALIGNED;
        int64_t bytes;
        if (!mul_ok(sz.state_bytes / N, static_cast<int64_t>(N) * cap, &bytes) ||
            bytes > (int64_t{1} << 62))
            return KDA_STATUS_INVALID_ARGUMENT;
        const Range r_s = range_of(snaps, bytes);
        for (const Range& in : inputs)
            if (overlaps(r_s, in)) return KDA_STATUS_INVALID_ARGUMENT;
        if (overlaps(r_s, r_gp) || overlaps(r_s, r_bp)) return KDA_STATUS_INVALID_ARGUMENT;
        if (overlaps(r_s, r_o) || overlaps(r_s, r_hT) || overlaps(r_s, r_ws))
            return KDA_STATUS_INVALID_ARGUMENT;
    }
    // the per-chunk state record (the two-pass path: resolve() checked)
    void* rec = options ? options->chunk_states : nullptr;
    if (rec) {
        if (snap != 0) return KDA_STATUS_INVALID_ARGUMENT;
        if (!aligned16(rec)) return KDA_STATUS_MISALIGNED;
        const Range r_c = range_of(rec, chunk_states_bytes(total_T, N, H));
        for (const Range& in : inputs)
            if (overlaps(r_c, in)) return KDA_STATUS_INVALID_ARGUMENT;
        if (overlaps(r_c, r_gp) || overlaps(r_c, r_bp) || overlaps(r_c, r_o) ||
            overlaps(r_c, r_hT) || overlaps(r_c, r_ws))
            return KDA_STATUS_INVALID_ARGUMENT;
    }

    kda::PrefillArgs a = shape_args(total_T, N, H, d_k, d_v, dtype);
    a.gate = gate;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.h0 = h0; a.cu_seqlens = cu_seqlens; a.o = o; a.hT = hT;
    a.order = static_cast<int32_t*>(workspace);
    a.scale = scale;
    a.snapshots = rec ? static_cast<float*>(rec) : snaps;
    a.snap_tokens = rec ? 64 : snaps ? snap : 0;
    a.snap_cap = rec ? -1 : cap;                   // < 0: the compact per-chunk record
    a.fe = fe;
    a.max_seqlen = options ? options->max_seqlen : 0;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (use_scratch) {
        const int ss = scratch_of(s, &workspace);
        if (ss != KDA_STATUS_OK) return ss;
        a.order = static_cast<int32_t*>(workspace);
    }
    hipError_t e = hipSuccess;
    switch (pl.path) {
        case KDA_PATH_VECTOR:
            if (kda::launch_plan(a, s) != hipSuccess) return KDA_STATUS_HIP_ERROR;
            e = kda::launch_prefill_valu(a, s);
            break;
        case KDA_PATH_MATRIX:
            if (kda::launch_plan(a, s) != hipSuccess) return KDA_STATUS_HIP_ERROR;
            e = kda::launch_prefill_mfma(a, pl.R, s);
            break;
        default:
            e = kda::launch_prefill_wy(a, pl.R, pl.L_b,
                                       static_cast<uint8_t*>(workspace) + plan_bytes(N), s);
            break;
    }
    return e == hipSuccess ? KDA_STATUS_OK : KDA_STATUS_HIP_ERROR;
}
}  // namespace

extern "C" {

int kda_fwd_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, const float* h0, const int32_t* cu_seqlens,
                    int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                    int32_t dtype, float scale, void* o, float* hT, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return kda_fwd_prefill_ex(q, k, v, log_alpha, beta, h0, cu_seqlens, total_T, N, H, d_k,
                              d_v, dtype, scale, o, hT, workspace, workspace_bytes, nullptr,
                              stream);
}

}  // extern "C"

namespace {
// Shared validation and launch of the decode entry points.  m = 0 is the
// single-step call (tokens [N][H][.], o required); m >= 1 is the
// several-token call (tokens [N][m][H][.]).
int decode_call(const void* q, const void* k, const void* v, const float* log_alpha,
                const float* beta, float* S, int32_t N, int32_t m, int32_t H, int32_t d_k,
                int32_t d_v, int32_t dtype, float scale, void* o, int32_t gate,
                const int32_t* index, int32_t num_states, const int32_t* lengths,
                bool write_state, const kda_front_end* front, void* stream) {
    const int32_t nstates = index ? num_states : N;
    if (nstates < 1 || m < 0 || N < 1) return KDA_STATUS_INVALID_ARGUMENT;
    int64_t tokens = N;
    if (m > 0 && !mul_ok(N, m, &tokens)) return KDA_STATUS_INVALID_ARGUMENT;
    Sizes sz;
    const int st = check_sizes(tokens, N, H, d_k, d_v, dtype, gate, &sz);
    if (st != KDA_STATUS_OK) return st;
    Sizes pool;   // the state pool: nstates states
    if (check_sizes(0, nstates, H, d_k, d_v, dtype, gate, &pool) != KDA_STATUS_OK)
        return KDA_STATUS_INVALID_ARGUMENT;
    if (!std::isfinite(scale)) return KDA_STATUS_INVALID_ARGUMENT;
    kda::FrontEnd fe;
    bool la_needed, beta_needed;
    Range r_gp, r_bp;
    const int fs = check_front(front, gate, log_alpha, beta, tokens, H, d_k, &fe, &la_needed,
                               &beta_needed, &r_gp, &r_bp);
    if (fs != KDA_STATUS_OK) return fs;
    if (!q || !k || !v || (beta_needed && !beta) || !S) return KDA_STATUS_INVALID_ARGUMENT;
    if (!o && (m == 0 || !write_state)) return KDA_STATUS_INVALID_ARGUMENT;   // nothing to do
    const int gs = check_gate_ptr(gate, log_alpha, la_needed);
    if (gs != KDA_STATUS_OK) return gs;
    if (gate == KDA_GATE_NONE) log_alpha = nullptr;   // never read
    const void* ptrs[] = {q, k, v, S, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_STATUS_MISALIGNED;
    if (!aligned4(beta) || !aligned4(index) || !aligned4(lengths)) return KDA_STATUS_MISALIGNED;
    const Range r_o = range_of(o, o ? sz.v_bytes : 0);
    const Range r_S = range_of(S, pool.state_bytes);
    const Range others[] = {range_of(q, sz.qk_bytes),      range_of(k, sz.qk_bytes),
                            range_of(v, sz.v_bytes),       range_of(log_alpha, sz.la_bytes),
                            range_of(beta, sz.beta_bytes), range_of(index, index ? N * 4 : 0),
                            range_of(lengths, lengths ? N * 4 : 0)};
    for (const Range& in : others)
        if (overlaps(r_o, in) || overlaps(r_S, in)) return KDA_STATUS_INVALID_ARGUMENT;
    for (const Range& in : {r_gp, r_bp})
        if (overlaps(r_o, in) || overlaps(r_S, in)) return KDA_STATUS_INVALID_ARGUMENT;
    if (overlaps(r_o, r_S)) return KDA_STATUS_INVALID_ARGUMENT;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.S = S; a.o = o;
    a.state_index = index; a.num_states = nstates;
    a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.gate = gate;
    a.dtype_f32 = dtype == KDA_DTYPE_F32;
    a.scale = scale;
    a.m = m;
    a.lengths = lengths;
    a.write_state = write_state;
    a.fe = fe;
    if (kda::launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_STATUS_HIP_ERROR;
    return KDA_STATUS_OK;
}
}  // namespace

extern "C" {

int kda_decode_step_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                       const float* beta, float* S, int32_t N, int32_t H, int32_t d_k,
                       int32_t d_v, int32_t dtype, float scale, void* o,
                       const kda_decode_options* options, void* stream) {
    const int32_t gate = options ? options->gate : KDA_GATE_CHANNEL;
    const int32_t* index = options ? options->state_index : nullptr;
    return decode_call(q, k, v, log_alpha, beta, S, N, 0, H, d_k, d_v, dtype, scale, o, gate,
                       index, options ? options->num_states : 0, nullptr, true,
                       options ? &options->front : nullptr, stream);
}

int kda_decode_multi(const void* q, const void* k, const void* v, const float* log_alpha,
                     const float* beta, float* S, int32_t N, int32_t m, int32_t H, int32_t d_k,
                     int32_t d_v, int32_t dtype, float scale, void* o,
                     const kda_decode_multi_options* options, void* stream) {
    if (m < 1) return KDA_STATUS_INVALID_ARGUMENT;
    const int32_t gate = options ? options->gate : KDA_GATE_CHANNEL;
    const int32_t* index = options ? options->state_index : nullptr;
    return decode_call(q, k, v, log_alpha, beta, S, N, m, H, d_k, d_v, dtype, scale, o, gate,
                       index, options ? options->num_states : 0,
                       options ? options->lengths : nullptr,
                       options ? options->write_state != 0 : true,
                       options ? &options->front : nullptr, stream);
}

int kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, float* S, int32_t N, int32_t H, int32_t d_k,
                    int32_t d_v, int32_t dtype, float scale, void* o, void* stream) {
    return kda_decode_step_ex(q, k, v, log_alpha, beta, S, N, H, d_k, d_v, dtype, scale, o,
                              nullptr, stream);
}


// ---- gradients of the prefill
static int bwd_block_chunks(int64_t total_T, int32_t N, int32_t H,
                            const kda_bwd_options* options, int* L_b) {
    const int32_t blk = options ? options->block_chunks : 0;
    const int64_t msl = options ? options->max_seqlen : 0;
    if (blk < 0 || msl < 0) return KDA_STATUS_INVALID_ARGUMENT;
    const int64_t seq_bound = msl > 0 && msl < total_T ? msl : total_T;
    *L_b = blk > 0 ? blk : kda::bwd_default_block_chunks(seq_bound, N, H);
    int64_t chunks;
    if (!mul_ok(static_cast<int64_t>(N) * H, *L_b, &chunks) || chunks >= (int64_t{1} << 31))
        return KDA_STATUS_INVALID_ARGUMENT;
    return KDA_STATUS_OK;
}

size_t kda_bwd_workspace_bytes(int64_t total_T, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                               int32_t dtype, const kda_bwd_options* options) {
    Sizes sz;
    if (check_sizes(total_T, N, H, d_k, d_v, dtype, options ? options->gate : 0, &sz) !=
        KDA_STATUS_OK)
        return 0;
    if (d_k != 128 || d_v != 128 || dtype != KDA_DTYPE_BF16 || !bwd_shape_ok(N, H)) return 0;
    int L_b;
    if (bwd_block_chunks(total_T, N, H, options, &L_b) != KDA_STATUS_OK) return 0;
    kda::FrontEnd fe;
    bool la_needed, beta_needed;
    Range r_gp, r_bp;
    const int32_t gate = options ? options->gate : KDA_GATE_CHANNEL;
    if (check_front(options ? &options->front : nullptr, gate, nullptr, nullptr, total_T, H, d_k,
                    &fe, &la_needed, &beta_needed, &r_gp, &r_bp) != KDA_STATUS_OK)
        return 0;
    const bool states = options && options->chunk_states;
    return kda::bwd_workspace_bytes(total_T, N, H, L_b, gate, fe, states);
}

int kda_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
            const float* beta, const float* h0, const int32_t* cu_seqlens, int64_t total_T,
            int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, float scale,
            const void* dO, const float* dhT, void* dq, void* dk, void* dv, float* dlog_alpha,
            float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
            const kda_bwd_options* options, void* stream) {
    const int32_t gate = options ? options->gate : KDA_GATE_CHANNEL;
    Sizes sz;
    const int st = check_sizes(total_T, N, H, d_k, d_v, dtype, gate, &sz);
    if (st != KDA_STATUS_OK) return st;
    if (d_k != 128 || d_v != 128 || dtype != KDA_DTYPE_BF16 || !bwd_shape_ok(N, H))
        return KDA_STATUS_UNSUPPORTED;
    if (!std::isfinite(scale) || !cu_seqlens) return KDA_STATUS_INVALID_ARGUMENT;
    void* aux = options ? options->aux_stream : nullptr;
    if (aux && aux == stream) return KDA_STATUS_INVALID_ARGUMENT;
    const bool any = total_T > 0;
    kda::FrontEnd fe;
    bool la_needed, beta_needed;
    Range r_gp, r_bp;
    const int fs = check_front(options ? &options->front : nullptr, gate, log_alpha, beta, total_T,
                               H, d_k, &fe, &la_needed, &beta_needed, &r_gp, &r_bp);
    if (fs != KDA_STATUS_OK) return fs;
    if (any && (!q || !k || !v || (beta_needed && !beta) || !dO || !dq || !dk || !dv || !dbeta))
        return KDA_STATUS_INVALID_ARGUMENT;
    int gs = la_needed ? check_gate_ptr(gate, log_alpha, any) : KDA_STATUS_OK;
    if (gs == KDA_STATUS_OK) gs = check_gate_ptr(gate, dlog_alpha, any);
    if (gs != KDA_STATUS_OK) return gs;
    if (gate == KDA_GATE_NONE) { log_alpha = nullptr; dlog_alpha = nullptr; }
    const void* ptrs[] = {q, k, v, h0, dO, dhT, dq, dk, dv, dh0, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_STATUS_MISALIGNED;
    if (!aligned4(beta) || !aligned4(dbeta) || !aligned4(cu_seqlens)) return KDA_STATUS_MISALIGNED;
    int L_b;
    const int bs = bwd_block_chunks(total_T, N, H, options, &L_b);
    if (bs != KDA_STATUS_OK) return bs;
    const void* states = options ? options->chunk_states : nullptr;
    if (states && !aligned16(states)) return KDA_STATUS_MISALIGNED;
    const size_t need = kda::bwd_workspace_bytes(total_T, N, H, L_b, gate, fe, states != nullptr);

    // no output may overlap an input, another output or the workspace
    const Range inputs[] = {range_of(q, sz.qk_bytes),      range_of(k, sz.qk_bytes),
                            range_of(v, sz.v_bytes),       range_of(log_alpha, sz.la_bytes),
                            range_of(beta, sz.beta_bytes), range_of(cu_seqlens, (N + 1) * 4),
                            range_of(h0, h0 ? sz.state_bytes : 0),
                            range_of(dO, sz.v_bytes),      range_of(dhT, dhT ? sz.state_bytes : 0),
                            r_gp,                          r_bp,
                            range_of(states, states ? chunk_states_bytes(total_T, N, H) : 0)};
    const Range outputs[] = {range_of(dq, sz.qk_bytes),     range_of(dk, sz.qk_bytes),
                             range_of(dv, sz.v_bytes),      range_of(dlog_alpha, sz.la_bytes),
                             range_of(dbeta, sz.beta_bytes), range_of(dh0, dh0 ? sz.state_bytes : 0),
                             range_of(workspace, static_cast<int64_t>(need))};
    const int nout = sizeof(outputs) / sizeof(outputs[0]);   // the workspace last
    for (int i = 0; i < nout - 1; ++i) {
        for (const Range& in : inputs)
            if (overlaps(outputs[i], in)) return KDA_STATUS_INVALID_ARGUMENT;
        for (int j = i + 1; j < nout - 1; ++j)
            if (overlaps(outputs[i], outputs[j])) return KDA_STATUS_INVALID_ARGUMENT;
    }
    if (workspace_bytes < need || !workspace) return KDA_STATUS_WORKSPACE_TOO_SMALL;
    for (int i = 0; i < nout - 1; ++i)
        if (overlaps(outputs[i], outputs[nout - 1])) return KDA_STATUS_INVALID_ARGUMENT;
    for (const Range& in : inputs)
        if (overlaps(outputs[nout - 1], in)) return KDA_STATUS_INVALID_ARGUMENT;

    kda::BackwardArgs a{};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.h0 = h0;
    a.cu_seqlens = cu_seqlens; a.dO = dO; a.dhT = dhT;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta; a.dh0 = dh0;
    a.total_T = total_T; a.N = N; a.H = H; a.gate = gate; a.scale = scale; a.fe = fe;
    a.states = states;
    a.max_seqlen = options ? options->max_seqlen : 0;
    a.aux = static_cast<hipStream_t>(aux);
    if (aux) {
        // the second stream must belong to the device of the caller's stream
        int d0 = -1, d1 = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &d0) != hipSuccess ||
            hipStreamGetDevice(a.aux, &d1) != hipSuccess)
            return KDA_STATUS_HIP_ERROR;
        if (d0 != d1) return KDA_STATUS_INVALID_ARGUMENT;
    }
    if (kda::launch_backward(a, L_b, workspace, static_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_STATUS_HIP_ERROR;
    return KDA_STATUS_OK;
}

}  // extern "C"

