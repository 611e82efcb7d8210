/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward pass.
 *
 * The operation.  Kimi Delta Attention (KDA) keeps one fixed-size state per
 * head and updates it once per token with a per-key-channel gated delta
 * rule:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t ,        alpha_t = exp(log_alpha_t)
 * i.e. decay every key channel of the state, predict the value stored for
 * k_t, scale the prediction error by beta_t, write it back along k_t, and
 * read the corrected state with the query.  Defined in "Kimi Delta
 * Attention: la atencion lineal detras de Kimi K2 y Qwen3", section "Cómo
 * funciona Kimi Delta Attention paso a paso" (the kda_step listing and the
 * flowchart); the per-channel gate is what "Cos'è Kimi Delta Attention
 * (KDA)?" (section "Gating per canale: cosa rende KDA diverso") sets apart
 * from Gated DeltaNet.  That listing scales the query by 1/sqrt(d_k); here
 * the scale is an argument and callers pass 1/sqrt(d_k) for that reading.
 * Keys are expected to be L2-normalised by the caller (the first page's
 * notes on key normalisation explain why the delta rule needs it).
 *
 * Gate variants.  The same recurrence with a coarser gate gives the two
 * models the pages compare KDA with: Gated DeltaNet, whose gate is one
 * scalar per (token, head) shared by every key channel ("Cos'è Kimi Delta
 * Attention (KDA)?", section "Gating per canale: cosa rende KDA diverso"
 * and its table), and DeltaNet, the delta rule with no decay at all
 * (alpha = 1) ("Kimi Delta Attention: la atencion lineal detras de Kimi K2
 * y Qwen3", section "DeltaNet, Gated DeltaNet y KDA: tabla comparativa").  The gate option of the _ex entry points selects the
 * layout of log_alpha (enum kda_gate); the kernels broadcast a scalar gate
 * over the key channels when they load it, so a Gated DeltaNet call gives
 * bitwise the result of a KDA call whose gate repeats that scalar.
 *
 * Layouts.  Every tensor is dense, contiguous, row-major:
 *     q, k        [total_T][H][d_k]     dtype (bf16 or fp32)
 *     v, o        [total_T][H][d_v]     dtype
 *     log_alpha   [total_T][H][d_k]     fp32, expected <= 0 (KDA_GATE_CHANNEL;
 *                 [total_T][H] for KDA_GATE_HEAD, not read for KDA_GATE_NONE)
 *     beta        [total_T][H]          fp32
 *     h0, hT, S   [N][H][d_k][d_v]      fp32 (d_v contiguous)
 *     cu_seqlens  [N+1]                 int32, DEVICE memory
 * A batch of N sequences is packed along the token axis: sequence n owns
 * tokens cu_seqlens[n] .. cu_seqlens[n+1]-1.  The state is always fp32.
 *
 * Ownership and execution.  The caller allocates every buffer (device
 * memory), including the prefill workspace, and every stream.  The library
 * keeps no global mutable state, allocates no device memory and never
 * synchronises: each call only enqueues kernels on `stream` (a
 * hipStream_t; NULL = the default stream) and returns.  The one call that
 * can use a second stream, kda_bwd, takes it from the caller
 * (kda_bwd_options.aux_stream) and orders the two with HIP events it
 * creates and releases within the call.  The one exception to "no state":
 * kda_fwd_prefill_noalloc, for callers that cannot allocate, works in a
 * static device array the library keeps on each GPU (see there).  Faults inside those kernels surface at the caller's next
 * synchronisation.  Calls on different streams may run concurrently if
 * their output buffers do not overlap.
 *
 * Errors.  Each entry point returns a kda_status value.  Every argument
 * check listed below happens on the host before any HIP call, so a
 * rejected call has no effect on the device.  Values inside device buffers
 * are NOT checked (that would need a synchronisation): cu_seqlens must be
 * 0 = c_0 <= c_1 <= ... <= c_N = total_T, and inputs must be finite.
 * A violated device-side precondition gives undefined values confined to
 * the sequences it touches; it never writes outside the caller's buffers
 * for sequences whose cu_seqlens entries lie inside [0, total_T].
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum kda_status {
    KDA_STATUS_OK = 0,
    KDA_STATUS_INVALID_ARGUMENT = 1,   /* null required pointer, bad size,
                                          size overflow, bad aliasing,
                                          non-finite scale */
    KDA_STATUS_UNSUPPORTED = 2,        /* d_k or d_v not in {16,32,64,128},
                                          unknown dtype */
    KDA_STATUS_MISALIGNED = 3,         /* a tensor pointer is not 16-byte
                                          aligned (beta, cu_seqlens: 4) */
    KDA_STATUS_WORKSPACE_TOO_SMALL = 4,
    KDA_STATUS_HIP_ERROR = 5           /* a kernel launch was refused */
};

/* Element type of q, k, v and o.  The state, log_alpha and beta are fp32. */
enum kda_dtype {
    KDA_DTYPE_BF16 = 0,
    KDA_DTYPE_F32 = 1
};

/* Layout of the gate log_alpha (see "Gate variants" above). */
enum kda_gate {
    KDA_GATE_CHANNEL = 0,  /* KDA: one gate per key channel, [..][H][d_k] */
    KDA_GATE_HEAD = 1,     /* Gated DeltaNet: one gate per (token, head),
                              [..][H], applied to every key channel */
    KDA_GATE_NONE = 2      /* DeltaNet: alpha = 1; log_alpha is not read and
                              may be NULL */
};

/* Which kernel family computes a prefill. */
enum kda_path {
    KDA_PATH_AUTO = 0,     /* a matrix path when supported (two-pass for
                              fewer than 128 (sequence, head) pairs, fused
                              otherwise), else the vector path */
    KDA_PATH_VECTOR = 1,   /* fp32 vector arithmetic, chunks of 32 tokens;
                              any supported dtype and head dimensions */
    KDA_PATH_MATRIX = 2,   /* bf16 matrix cores, fp32 accumulation and
                              state, chunks of 64 tokens, one fused kernel
                              per (sequence, head, value tile); bf16 and
                              d_k = 128 */
    KDA_PATH_MATRIX_TWO_PASS = 3
                           /* the same arithmetic in two kernels: a
                              chunk-parallel pass builds each chunk's
                              state-independent operands into the
                              workspace, a serial pass carries the state;
                              for few long sequences.  bf16, d_k = 128 */
};

/*
 * The fused input front-end: raw projections go in, the kernels apply the
 * activations while they stage the inputs.  Every part is optional:
 *   l2norm_qk  nonzero: q and k are divided, per (token, head), by
 *              max(||x||_2, 1e-6) -- the unit keys the delta rule needs
 *              ("Kimi Delta Attention: la atencion lineal detras de Kimi K2
 *              y Qwen3", notes on key normalisation);
 *   gate_pre   DEVICE bf16 pre-activations x in log_alpha's layout for the
 *              call's gate (KDA: [tokens][H][d_k], 16-byte aligned; Gated
 *              DeltaNet: [tokens][H], 2-byte aligned), replacing log_alpha,
 *              which must then be NULL: log_alpha = -gate_scale *
 *              softplus(x), so alpha is in (0, 1] for gate_scale >= 0;
 *   beta_pre   DEVICE bf16 [tokens][H] pre-activations y (2-byte aligned),
 *              replacing beta, which must then be NULL: beta = sigmoid(y).
 * The pre-activations are bf16 whatever the dtype of q, k, v.  They cut a
 * prefill's input from 1540 to 1282 bytes per head-token at d = 128.
 */
typedef struct kda_front_end {
    int32_t l2norm_qk;
    float gate_scale;              /* finite, >= 0; used with gate_pre */
    const void *gate_pre;
    const void *beta_pre;
} kda_front_end;

/* Tuning options of kda_fwd_prefill_ex (zero-initialise for defaults). */
typedef struct kda_prefill_options {
    int32_t path;          /* a kda_path */
    int32_t value_tiles;   /* work-groups per (sequence, head), each owning
                              d_v / value_tiles state columns; 0 = automatic.
                              A power of two with 16 <= d_v / value_tiles
                              (<= 32 on the two-pass path).  Ignored by the vector
                              path, which always uses 32-column tiles
                              (16 when d_v = 16). */
    int32_t block_chunks;  /* two-pass path: chunks of every sequence per
                              pass pair (the workspace holds
                              N * H * block_chunks chunk slots of
                              55808 + 128 d_v bytes); 0 = automatic
                              (about 150 MiB of slots).  Ignored by the
                              other paths. */
    int32_t gate;          /* a kda_gate (0 = KDA_GATE_CHANNEL) */
    int32_t snapshot_tokens;   /* 0 = no snapshots; else a positive multiple
                                  of 64: the state after every
                                  snapshot_tokens tokens of each sequence is
                                  written to snapshots (for prefix caching:
                                  a snapshot can seed a later call as its
                                  h0) */
    int32_t snapshot_capacity; /* snapshots kept per sequence (>= 1 when
                                  snapshot_tokens > 0) */
    float *snapshots;          /* DEVICE [N][snapshot_capacity][H][d_k][d_v]
                                  fp32, 16-byte aligned: snapshot j of
                                  sequence n is the state after its first
                                  (j+1) * snapshot_tokens tokens, for those
                                  j < snapshot_capacity that fit in the
                                  sequence; other entries are not written.
                                  May not overlap any other buffer. */
    kda_front_end front;       /* the fused input front-end (all off when
                                  zeroed); every path */
    void *chunk_states;        /* DEVICE, kda_chunk_states_bytes bytes,
                                  16-byte aligned, or NULL: the start state
                                  of every chunk of 64 tokens after a
                                  sequence's first (bf16), recorded for a
                                  later kda_bwd on the same inputs, which
                                  then skips recomputing the forward pass.
                                  Two-pass path, bf16, d_k = d_v = 128;
                                  not with snapshot_tokens; no overlap with
                                  any other buffer. */
    int64_t max_seqlen;        /* 0 = unknown; else at least the longest
                                  sequence of the call (cu_seqlens lives in
                                  device memory, so only the caller knows
                                  it).  The two-pass path then runs its
                                  block loop over that many tokens instead
                                  of total_T: a batch of N equal sequences
                                  launches 1/N of the blocks.  A sequence
                                  longer than max_seqlen (a violated device
                                  precondition) gets a NaN final state and
                                  its outputs past max_seqlen are not
                                  written.  Ignored by the other paths. */
} kda_prefill_options;


/* Options of kda_decode_step_ex (zero-initialise for defaults). */
typedef struct kda_decode_options {
    int32_t gate;                  /* a kda_gate (0 = KDA_GATE_CHANNEL) */
    int32_t num_states;            /* states in S when state_index is set */
    const int32_t *state_index;    /* DEVICE [N], or NULL: sequence n reads
                                      and updates state S[state_index[n]]
                                      (S is [num_states][H][d_k][d_v]); NULL
                                      means S[n] (S is [N][H][d_k][d_v]).
                                      A sequence whose index lies outside
                                      [0, num_states) is skipped: its state
                                      is not touched and its o not written.
                                      Indices of one call must be distinct
                                      (two sequences updating one state
                                      race). */
    kda_front_end front;           /* the fused input front-end, as for the
                                      prefill (tokens = N) */
} kda_decode_options;

/* Options of kda_decode_multi (zero-initialise, then set write_state, for
 * the common call). */
typedef struct kda_decode_multi_options {
    int32_t gate;                  /* a kda_gate (0 = KDA_GATE_CHANNEL) */
    int32_t num_states;            /* states in S when state_index is set */
    const int32_t *state_index;    /* DEVICE [N] or NULL: the state map of
                                      kda_decode_options, same rules */
    const int32_t *lengths;        /* DEVICE [N] or NULL: sequence n applies
                                      its first clamp(lengths[n], 0, m)
                                      tokens; NULL means all m */
    int32_t write_state;           /* nonzero: each sequence's state is
                                      overwritten with the state after its
                                      applied tokens (left as it was when it
                                      applies none); zero: S is only read */
    kda_front_end front;           /* the fused input front-end, per token
                                      (zero = none); as for kda_decode_step_ex */
} kda_decode_multi_options;

/* Options of kda_bwd (zero-initialise for defaults). */
typedef struct kda_bwd_options {
    int32_t gate;                  /* a kda_gate (0 = KDA_GATE_CHANNEL) */
    int32_t block_chunks;          /* chunks of 64 tokens per backward block
                                      (0 = automatic) */
    kda_front_end front;           /* the fused input front-end the forward
                                      used (zero = none); see kda_bwd */
    const void *chunk_states;      /* DEVICE or NULL: the record a
                                      kda_fwd_prefill_ex call wrote on these
                                      same inputs (options.chunk_states);
                                      the forward pass is then not
                                      recomputed */
    int64_t max_seqlen;            /* 0 = unknown; else at least the longest
                                      sequence, as for the prefill: the block
                                      loop covers that many tokens.  A
                                      longer sequence gets NaN in dh0 (when
                                      requested) and unwritten gradients
                                      past max_seqlen. */
    void *aux_stream;              /* a second hipStream_t of the same
                                      device, or NULL.  Set: the per-block
                                      operand pass and the serial
                                      state-adjoint pass run on it, beside
                                      the gradient pass on `stream` (the
                                      call creates and destroys its own HIP
                                      events to order the two; no device
                                      memory).  NULL: the whole call runs
                                      in order on `stream`.  The results are
                                      the same bits either way. */
} kda_bwd_options;

/* Version of this ABI; bumped whenever a signature or a layout changes. */
int kda_abi_version(void);

/*
 * Bytes of the per-chunk state record (kda_prefill_options.chunk_states,
 * kda_bwd_options.chunk_states) for these sizes: one bf16 d_k x d_v state
 * per (chunk index, head) over N + ceil(total_T / 64) + 1 chunk indices.
 * 0 unless d_k = d_v = 128, or for sizes kda_fwd_prefill would reject.
 */
size_t kda_chunk_states_bytes(int64_t total_T, int32_t N, int32_t H, int32_t d_k,
                              int32_t d_v);

/* Human-readable text for a status code (static storage; never NULL). */
const char *kda_status_string(int status);

/*
 * Bytes of device workspace kda_fwd_prefill needs for these sizes: the
 * sequence scheduling table, plus, when the two-pass path is chosen, one
 * block of per-(chunk, head) operand slots and a copy of the states.  Pure
 * host arithmetic; returns 0 for arguments kda_fwd_prefill would reject.
 */
size_t kda_fwd_prefill_workspace_bytes(int64_t total_T, int32_t N, int32_t H,
                                       int32_t d_k, int32_t d_v, int32_t dtype);

/* The same for kda_fwd_prefill_ex with these options (NULL = defaults). */
size_t kda_fwd_prefill_workspace_bytes_ex(int64_t total_T, int32_t N, int32_t H,
                                          int32_t d_k, int32_t d_v, int32_t dtype,
                                          const kda_prefill_options *options);

/*
 * Chunked prefill over a packed batch of N sequences.
 *
 * Computes o for every token and, if hT != NULL, the state after each
 * sequence's last token (hT[n] = h0[n], or zeros, for an empty sequence).
 * h0 == NULL means a zero initial state.  hT may be the same buffer as h0
 * (each state is read before it is written by the same work-group); any
 * other overlap between an output (o, hT) and any input is rejected.
 *
 * Precision: bf16 inputs use bf16 matrix-core products with fp32
 * accumulation and an fp32 state; fp32 inputs use fp32 arithmetic
 * throughout.  o is written in the input dtype (round to nearest even).
 * Gate range: every path takes any log_alpha <= 0 (any alpha in (0, 1]).
 * Within a chunk the kernels normally form the decays as
 * exp(g) * exp(-g) of the chunk's cumulative gate g, which stays inside
 * fp32 while |g| <= 80 (natural log).  A chunk beyond that (a channel whose
 * gates sum below -80 over the chunk, e.g. per-token gates below -1.25 on
 * the matrix paths' 64-token chunks) takes another form for its
 * decay-weighted products, at a higher cost for that chunk only:
 *  - on the matrix paths, when each 16-row block of the chunk keeps its own
 *    gate sum within 80: the blocked form, matrix-core products again, with
 *    the decays factored through the cumulative gate before each row block
 *    (a two-pass prefill whose every chunk takes it runs about 1.3x longer,
 *    a fused one about 1.9x);
 *  - otherwise (and on the vector path, already beyond |g| = 16, from fp64
 *    cumulative gates): the exact pairwise form, each entry summed with its
 *    own factors exp(g_r - g_s) <= 1 (about 2.2x to 7x longer).
 * Positive log_alpha (outside the domain) is not checked; where it pushes a
 * row beyond the range on the fused path, that row's output is NaN.
 *
 * Requirements (else the status in brackets):
 *   N >= 1, H >= 1, total_T >= 0, sizes whose byte counts fit in int64
 *     [INVALID_ARGUMENT];
 *   q, k, v, log_alpha, beta, o non-NULL when total_T > 0; cu_seqlens
 *     non-NULL; scale finite [INVALID_ARGUMENT];
 *   d_k, d_v in {16, 32, 64, 128}; dtype a kda_dtype [UNSUPPORTED];
 *   q, k, v, log_alpha, h0, o, hT and workspace 16-byte aligned, beta and
 *     cu_seqlens 4-byte aligned [MISALIGNED];
 *   workspace_bytes >= kda_fwd_prefill_workspace_bytes(...) and workspace
 *     non-NULL if that is > 0 [WORKSPACE_TOO_SMALL].
 */
int kda_fwd_prefill(const void *q, const void *k, const void *v,
                    const float *log_alpha, const float *beta,
                    const float *h0, const int32_t *cu_seqlens,
                    int64_t total_T, int32_t N, int32_t H,
                    int32_t d_k, int32_t d_v, int32_t dtype, float scale,
                    void *o, float *hT,
                    void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * kda_fwd_prefill with explicit options (NULL = defaults).  Same arguments,
 * results and requirements as kda_fwd_prefill, plus:
 *   options->path not a kda_path, value_tiles invalid for the chosen path,
 *     block_chunks negative or too large, or gate not a kda_gate
 *     [INVALID_ARGUMENT];
 *   log_alpha: [total_T][H][d_k], 16-byte aligned (KDA_GATE_CHANNEL);
 *     [total_T][H], 4-byte aligned (KDA_GATE_HEAD); may be NULL
 *     (KDA_GATE_NONE) [INVALID_ARGUMENT, MISALIGNED];
 *   snapshot_tokens not 0 and not a positive multiple of 64, or set with
 *     snapshot_capacity < 1, snapshots NULL, a byte count that overflows,
 *     or snapshots overlapping another buffer [INVALID_ARGUMENT];
 *     snapshots not 16-byte aligned [MISALIGNED];
 *   chunk_states set together with snapshot_tokens, or overlapping another
 *     buffer [INVALID_ARGUMENT]; not 16-byte aligned [MISALIGNED]; with the
 *     vector or the fused matrix path, fp32 inputs, or d_k or d_v other
 *     than 128 [UNSUPPORTED] (the automatic path is then the two-pass one);
 *   a matrix path requested for fp32 inputs or d_k != 128 [UNSUPPORTED];
 *   workspace_bytes below kda_fwd_prefill_workspace_bytes_ex(..., options)
 *     [WORKSPACE_TOO_SMALL].
 * Every path computes the same chunked form of the recurrence with its own
 * chunk length and precision; results agree to the precision bound above.
 * The two matrix paths round their operands the same way but sum in
 * different orders, so they agree to that bound, not bitwise; two-pass
 * results do not depend on block_chunks (the state crosses blocks in fp32).
 */
int kda_fwd_prefill_ex(const void *q, const void *k, const void *v,
                       const float *log_alpha, const float *beta,
                       const float *h0, const int32_t *cu_seqlens,
                       int64_t total_T, int32_t N, int32_t H,
                       int32_t d_k, int32_t d_v, int32_t dtype, float scale,
                       void *o, float *hT,
                       void *workspace, size_t workspace_bytes,
                       const kda_prefill_options *options, void *stream);

/*
 * The allocation-free prefill: kda_fwd_prefill_ex with no workspace
 * argument, for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Its workspace is a static device array of KDA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends (the HIP
 * runtime places it when it loads the library's code on that GPU); its
 * device address is looked up once per device, on the first call there.
 * A call allocates nothing and never synchronises.
 *
 * Same arguments, results and requirements as kda_fwd_prefill_ex, except:
 *   the two-pass path with options->block_chunks = 0 takes the largest
 *     block length (up to its usual default) whose workspace fits the
 *     array; results do not depend on the block length;
 *   a call whose workspace does not fit the array (e.g. the two-pass path
 *     with N * H * (55808 + 128 d_v) bytes of one block's slots above it)
 *     [WORKSPACE_TOO_SMALL], before any HIP call;
 *   the array's address could not be looked up [HIP_ERROR].
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (no call needs them cleared): calls that overlap on one GPU --
 * on different streams, or from several host threads -- race on it and
 * must be serialised by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
int kda_fwd_prefill_noalloc(const void *q, const void *k, const void *v,
                            const float *log_alpha, const float *beta,
                            const float *h0, const int32_t *cu_seqlens,
                            int64_t total_T, int32_t N, int32_t H,
                            int32_t d_k, int32_t d_v, int32_t dtype, float scale,
                            void *o, float *hT,
                            const kda_prefill_options *options, void *stream);

/*
 * One decode step: one new token for each of N sequences.
 *
 * Inputs q, k [N][H][d_k], v [N][H][d_v] (dtype), log_alpha [N][H][d_k],
 * beta [N][H] (fp32).  The state S [N][H][d_k][d_v] (fp32) is read and
 * overwritten in place with the state after the token; o [N][H][d_v]
 * (dtype) receives the token's output.  This is exactly one token of the
 * recurrence above; chaining T calls equals a prefill over those T tokens.
 * o must not overlap any input or S.
 *
 * Requirements: N >= 1, H >= 1, all pointers non-NULL, scale finite
 * [INVALID_ARGUMENT]; d_k, d_v in {16, 32, 64, 128}, dtype a kda_dtype
 * [UNSUPPORTED]; q, k, v, log_alpha, S and o 16-byte aligned, beta 4-byte
 * aligned [MISALIGNED].
 */
int kda_decode_step(const void *q, const void *k, const void *v,
                    const float *log_alpha, const float *beta, float *S,
                    int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                    int32_t dtype, float scale, void *o, void *stream);

/*
 * kda_decode_step with options (NULL = defaults): the gate layout, and a
 * state map for serving, where the states of the running sequences sit in
 * slots of a larger pool (continuous batching).  Same arguments, results
 * and requirements as kda_decode_step, plus:
 *   options->gate not a kda_gate, or state_index set with num_states < 1
 *     [INVALID_ARGUMENT];
 *   log_alpha as for kda_fwd_prefill_ex with that gate [INVALID_ARGUMENT,
 *     MISALIGNED];
 *   state_index 4-byte aligned [MISALIGNED]; S holds num_states states when
 *     state_index is set, and no output may overlap state_index
 *     [INVALID_ARGUMENT].
 */
int kda_decode_step_ex(const void *q, const void *k, const void *v,
                       const float *log_alpha, const float *beta, float *S,
                       int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                       int32_t dtype, float scale, void *o,
                       const kda_decode_options *options, void *stream);

/*
 * Several decode tokens per sequence in one pass over the states: m tokens
 * for each of N sequences, applied in order, each one token of the
 * recurrence above exactly as kda_decode_step applies it.  This serves the
 * speculative decoding that "Kimi Linear acaba de superar a la atención
 * completa en sus propios términos" (section "Qué observar tras el
 * lanzamiento de Kimi Linear") lists among the serving features KDA has to
 * keep correct: one call verifies m draft tokens (o given, write_state = 0:
 * the outputs of all m, the states untouched) and a second commits the
 * accepted prefix (o = NULL, write_state = 1, lengths = tokens accepted per
 * sequence).  Each state is read once per call and written at most once,
 * whatever m is.
 *
 * Inputs q, k [N][m][H][d_k], v [N][m][H][d_v] (dtype), log_alpha laid out
 * per options->gate over the same N*m tokens, beta [N][m][H] (fp32).  S as
 * for kda_decode_step_ex.  o [N][m][H][d_v] (dtype) or NULL receives the
 * outputs of the applied tokens; rows of tokens a sequence does not apply,
 * and every row of a skipped sequence, are left unwritten.
 *
 * Requirements: m >= 1, and o != NULL or write_state != 0
 * [INVALID_ARGUMENT]; lengths 4-byte aligned [MISALIGNED] and no overlap of
 * an output with it [INVALID_ARGUMENT]; otherwise those of
 * kda_decode_step_ex over N*m tokens.
 */
int kda_decode_multi(const void *q, const void *k, const void *v,
                     const float *log_alpha, const float *beta, float *S,
                     int32_t N, int32_t m, int32_t H, int32_t d_k, int32_t d_v,
                     int32_t dtype, float scale, void *o,
                     const kda_decode_multi_options *options, void *stream);

/*
 * Bytes of device workspace kda_bwd needs for these sizes and options:
 * the start state of every chunk (one bf16 state per (chunk, head), so
 * 512 MiB per 16,384 head-chunks), the forward pass's operand block, and
 * three blocks of per-(chunk, head) backward operands (one filled while
 * the others are consumed); with the front-end, also the activated inputs it
 * produces (normalised q and k in bf16, log_alpha and beta in fp32, each
 * when its part is on; only whether options->front's pointers are set
 * matters here).  0 for arguments kda_bwd would reject.
 */
size_t kda_bwd_workspace_bytes(int64_t total_T, int32_t N, int32_t H,
                               int32_t d_k, int32_t d_v, int32_t dtype,
                               const kda_bwd_options *options);

/*
 * Gradients of the prefill: with L = <o, dO> + <hT, dhT> for the prefill
 * kda_fwd_prefill computes on these inputs, writes dL/dq, dL/dk, dL/dv
 * (dtype, the layouts of q, k, v), dL/dlog_alpha (fp32, the layout of
 * log_alpha for the gate in options), dL/dbeta [total_T][H] (fp32) and,
 * when dh0 != NULL, dL/dh0 [N][H][d_k][d_v] (fp32).  dhT == NULL means a
 * zero adjoint of the final states.  This is the backward pass of the
 * chunkwise training algorithm that "Kimi Linear acaba de superar a la
 * atención completa en sus propios términos" (section "Cómo Kimi Linear
 * utiliza una memoria recurrente más inteligente") credits for KDA's
 * training efficiency; the forward is recomputed inside the call, so only
 * the forward's inputs are needed.
 *
 * Requirements: those of kda_fwd_prefill for the shared inputs; dO
 * [total_T][H][d_v] (dtype) non-NULL when total_T > 0, as are dq, dk, dv,
 * dbeta, and dlog_alpha unless the gate is KDA_GATE_NONE
 * [INVALID_ARGUMENT]; d_k = d_v = 128 and dtype KDA_DTYPE_BF16
 * [UNSUPPORTED]; dO, dhT, dq, dk, dv, dh0, the workspace and a per-channel
 * dlog_alpha 16-byte aligned, dbeta and a per-head dlog_alpha 4-byte
 * aligned [MISALIGNED]; no output overlapping an input, another output or
 * the workspace [INVALID_ARGUMENT]; workspace_bytes at least
 * kda_bwd_workspace_bytes [WORKSPACE_TOO_SMALL].
 * Precision: bf16 matrix products with fp32 accumulation, fp32 states and
 * adjoints, as in the forward pass.  Gate range: the whole domain
 * (log_alpha <= 0, any finite value).  A chunk whose cumulative gate leaves
 * the factored form's range (|g| > 80, see kda_fwd_prefill) takes the
 * blocked or the exact pairwise form for its decay-weighted products, as in
 * kda_fwd_prefill, in the operand pass and in the gradient pass, at some
 * cost in time for that chunk only (every chunk at -3 per token, blocked:
 * about 1.3x).
 * Saved states (options->chunk_states): the record of the forward pass on
 * these inputs replaces its recomputation (the call then reads the record
 * and needs a smaller workspace); the record must come from a forward pass
 * on the same q, k, v, gates, beta, h0 and cu_seqlens (and, with the
 * front-end, the same front-end options).  16-byte aligned [MISALIGNED];
 * no output may overlap it [INVALID_ARGUMENT].
 * Front-end (options->front, as for kda_fwd_prefill_ex): q and k are the raw
 * inputs when l2norm_qk is set, and dq, dk the gradients with respect to
 * them; with gate_pre, log_alpha must be NULL and dlog_alpha (fp32, the
 * gate's layout) receives the gradient with respect to gate_pre; with
 * beta_pre, beta must be NULL and dbeta receives the gradient with respect
 * to beta_pre.  The activations are computed once ahead of the backward
 * (normalised q and k are stored in bf16), and the chain rule through them
 * is applied to the gradients afterwards.  Requirements and errors as for
 * kda_fwd_prefill_ex's front-end.
 * Streams: with options->aux_stream set, the per-block operand pass and
 * the serial state-adjoint pass run on that stream, ordered against
 * `stream` by per-call events, and the first work on it waits for
 * `stream`'s earlier work; all of the call's work is complete once `stream`
 * reaches the point after the call.  aux_stream must belong to the device
 * of `stream` [INVALID_ARGUMENT] and must not be `stream` itself.
 * d_k = d_v = 128, bf16 and H <= 16384 [UNSUPPORTED].
 */
int kda_bwd(const void *q, const void *k, const void *v,
            const float *log_alpha, const float *beta, const float *h0,
            const int32_t *cu_seqlens, int64_t total_T, int32_t N, int32_t H,
            int32_t d_k, int32_t d_v, int32_t dtype, float scale,
            const void *dO, const float *dhT, void *dq, void *dk, void *dv,
            float *dlog_alpha, float *dbeta, float *dh0,
            void *workspace, size_t workspace_bytes,
            const kda_bwd_options *options, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
