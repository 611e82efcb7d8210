// kda_internal.h -- argument bundles and launcher declarations shared by the
// host entry points (kda_api.cpp) and the kernel translation units.  Every
// launcher only enqueues work on the given stream; argument validation has
// already happened on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// layout of log_alpha: one gate per key channel, one per (token, head)
// shared by every channel, or none (alpha = 1; log_alpha not read)
enum GateMode : int { kGateChannel = 0, kGateHead = 1, kGateNone = 2 };

// The fused input front-end: each part is optional.
//   l2norm:   q and k are divided by max(||x||_2, kFrontEps) per (token, head)
//   gate_pre: bf16 pre-activations x in log_alpha's layout, which is then
//             unused: log_alpha = -gate_scale * softplus(x)
//   beta_pre: bf16 [tokens][H] pre-activations y: beta = sigmoid(y)
struct FrontEnd {
    const uint16_t* gate_pre = nullptr;   // bf16 bits
    const uint16_t* beta_pre = nullptr;   // bf16 bits
    float gate_scale = 0.f;
    bool l2norm = false;
    bool active() const { return l2norm || gate_pre || beta_pre; }
};
constexpr float kFrontEps = 1e-6f;

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    float* S;
    void* o;
    const int32_t* state_index;   // device [N] or null: sequence n uses S[state_index[n]]
    int32_t num_states;           // states in S when state_index is set
    int32_t N, H, d_k, d_v;
    int gate;                     // a GateMode
    bool dtype_f32;
    float scale;
    FrontEnd fe;
    // several tokens per sequence (m > 0; 0 = the single-step kernel):
    // tokens [N][m][H][.], lengths device [N] or null, o may be null
    int32_t m = 0;
    const int32_t* lengths = nullptr;
    bool write_state = true;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* h0;            // may be null (zero initial state)
    const int32_t* cu_seqlens;  // device, [N+1]
    void* o;
    float* hT;                  // may be null (not written)
    int32_t* order;             // device scratch [N]: sequences by length, longest first
    int64_t total_T;
    int32_t N, H, d_k, d_v;
    int gate;                   // a GateMode
    bool dtype_f32;
    float scale;
    // state snapshots: after every snap_tokens tokens of a sequence (a
    // multiple of 64), into snapshots[n][j][h] for j < snap_cap; null = none
    float* snapshots;
    int32_t snap_tokens, snap_cap;
    FrontEnd fe;
    // the longest sequence, or 0 (unknown: total_T); bounds the two-pass
    // block loop
    int64_t max_seqlen = 0;
    int64_t seq_bound() const {
        return max_seqlen > 0 && max_seqlen < total_T ? max_seqlen : total_T;
    }
};

// gradients of the prefill (bf16, d_k = d_v = 128): see backward.hip
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;     // per the gate layout; null without a gate
    const float* beta;
    const float* h0;            // may be null (zero initial state)
    const int32_t* cu_seqlens;  // device, [N+1]
    const void* dO;             // [total_T][H][d_v], the adjoint of o
    const float* dhT;           // may be null (zero adjoint of the final states)
    void* dq;
    void* dk;
    void* dv;
    float* dlog_alpha;          // per the gate layout; null without a gate
    float* dbeta;
    float* dh0;                 // may be null (not written)
    int64_t total_T;
    int32_t N, H;
    int gate;
    float scale;
    // the fused input front-end: q and k raw, log_alpha / beta null where
    // gate_pre / beta_pre stand in; dq, dk, dlog_alpha and dbeta are then
    // the gradients with respect to the raw inputs and pre-activations
    FrontEnd fe;
    // the per-chunk state record of a forward pass on these inputs, or null
    // (the forward pass is then recomputed into the workspace)
    const void* states = nullptr;
    // the longest sequence, or 0 (unknown: total_T); bounds the block loop
    int64_t max_seqlen = 0;
    // a second stream of the device for the operand and carry passes, or
    // null (the whole call in order on the caller's stream)
    hipStream_t aux = nullptr;
    int64_t seq_bound() const {
        return max_seqlen > 0 && max_seqlen < total_T ? max_seqlen : total_T;
    }
};
int bwd_default_block_chunks(int64_t seq_bound, int32_t N, int32_t H);
// the backward's buffers, after the front-end's activated inputs when fe is
// active
size_t bwd_workspace_bytes(int64_t total_T, int32_t N, int32_t H, int L_b, int gate,
                           const FrontEnd& fe, bool have_states);
hipError_t launch_backward(const BackwardArgs& a, int L_b, void* ws, hipStream_t stream);

// first element of snapshot j of (sequence n, head h): [N][snap_cap][H][d_k][d_v]
__host__ __device__ __forceinline__ float* snapshot_at(float* snapshots, int snap_cap, int H,
                                                       int64_t state_elems, int n, int j, int h) {
    return snapshots + ((static_cast<int64_t>(n) * snap_cap + j) * H + h) * state_elems;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_plan(const PrefillArgs& a, hipStream_t stream);

// fp32 vector path (any dtype and supported head dimensions)
hipError_t launch_prefill_valu(const PrefillArgs& a, hipStream_t stream);
// bf16 matrix-core path (d_k = 128); R value tiles per (sequence, head)
bool mfma_supported(const PrefillArgs& a);
int mfma_value_tiles(const PrefillArgs& a);
bool mfma_tiles_ok(int d_v, int R);
hipError_t launch_prefill_mfma(const PrefillArgs& a, int R, hipStream_t stream);
// bf16 two-pass matrix-core path (d_k = 128): a chunk-parallel prep kernel
// and a serial carry kernel, alternated over blocks of L_b chunks; the
// workspace holds one block of per-(chunk, head) slots plus a state copy
bool wy_supported(const PrefillArgs& a);
int wy_value_tiles(const PrefillArgs& a);
bool wy_tiles_ok(int d_v, int R);
int wy_default_block_chunks(int64_t seq_bound, int32_t N, int32_t H, int32_t d_v);
bool wy_block_chunks_ok(int32_t N, int32_t H, int L_b);
size_t wy_workspace_bytes(int32_t N, int32_t H, int32_t d_k, int32_t d_v, int L_b);
hipError_t launch_prefill_wy(const PrefillArgs& a, int R, int L_b, void* ws, hipStream_t stream);

}  // namespace kda
