/*
 * gdn.h -- C ABI of the MI355X (gfx950) GatedDeltaNet gated delta-rule library.
 *
 * Operation.  Per value head, the gated delta rule ("Qwen3.5-27B GPTQ Garbage
 * Inference -- Root Cause Analysis", section "Why abliteration failed on
 * Qwen3.5", item 3, with the delta read as the prediction error of the
 * decayed state):
 *     S_t = e^{g_t} S_{t-1} + beta_t (v_t - e^{g_t} S_{t-1} k_t) k_t^T
 *     o_t = scale * S_t q_t              (scale = d_k^{-1/2} by default)
 * where S is d_v x d_k.  The STORED state is H = S^T, fp32, laid out
 * [seq][h_v][d_k][d_v] with d_v contiguous ("[Feature] Add batch invariance
 * support to GDN_ATTN backend", review comment part "1. Recurrent state in
 * fp32": shape (batch, v_heads, k_head_dim, v_head_dim), fp32).
 *
 * Prologue (same page, part "3. The chunked delta-rule scan itself", (a)):
 * with conv_width = 4, every q|k|v channel c goes through a causal depthwise
 * convolution y_t[c] = b[c] + sum_{j=0..3} w[c][j] x_{t-3+j}[c] (w[c][3] hits
 * the newest token) followed by SiLU; history before a sequence start is the
 * given conv state (3 raw inputs per channel, oldest first) or zero, never
 * the previous packed sequence.  Then, with qk_l2norm = 1, q and k are
 * normalised per head: x / sqrt(sum x^2 + l2_eps).  Channel order is q | k | v,
 * each head-major: C = 2 h_k d_k + h_v d_v channels.
 *
 * GQA: value head h reads key head h / (h_v / h_k).
 *
 * Layout.  One layout only: time-first and packed ("Qwen3.5 FLA linear
 * attention tensor format mismatch", section "Root Cause": [B, T, H, D], not
 * head-first).  Sequences are concatenated and delimited by cu_seqlens, one
 * entry per sequence start plus the total ("[Feature] Add batch invariance
 * support to GDN_ATTN backend", commit messages: cu_seqlens = [0, len] per
 * sequence).  There is no batch dimension and no layout heuristic.
 *
 * Conventions.
 *  - All tensor pointers are DEVICE pointers, row-major, contiguous.  The
 *    gdn_problem struct is HOST memory and is read during the call only.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronises; work is enqueued on `stream` (a hipStream_t passed as
 *    void*, NULL = the null stream) and the call returns without waiting.
 *  - Argument errors return a negative status before any HIP call and leave
 *    every output untouched.  A failed launch returns GDN_ERR_HIP.
 *  - Device-side contents are preconditions, not checked: cu_seqlens
 *    non-decreasing with cu_seqlens[0] = 0 and cu_seqlens[N] = total_tokens;
 *    state indices in range and distinct (except -1).  NaN/Inf propagate.
 *  - Batch invariance: a sequence's outputs and final states are bit-identical
 *    whatever other sequences share the call; kernel choice depends only on
 *    (d_k, d_v, qkv_dtype, out_dtype), never on N, lengths or totals.
 *  - Exponentials are only taken of non-positive decay differences when
 *    g <= 0 (a log decay); positive g is accepted with no overflow guarantee.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_dtype {
    GDN_F32 = 0,  /* IEEE fp32 */
    GDN_BF16 = 1  /* bfloat16 (8-bit exponent, 7-bit mantissa) */
} gdn_dtype;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
    GDN_ERR_DTYPE = -3,       /* dtype value not in gdn_dtype */
    GDN_ERR_UNSUPPORTED = -4, /* valid request this build has no kernel for */
    GDN_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
    GDN_ERR_HIP = -6,         /* a kernel launch failed */
    GDN_ERR_ALIAS = -7,       /* an output overlaps a buffer it must not */
    GDN_ERR_SCRATCH = -8      /* the problem needs more than the static scratch
                               * of gdn_prefill_varlen_noalloc */
} gdn_status;

typedef struct gdn_problem {
    int32_t num_seqs;      /* N >= 0: sequences (prefill) or slots (decode) */
    int64_t total_tokens;  /* prefill: cu_seqlens[N]; decode: must equal N */
    int32_t h_k, h_v;      /* key and value heads, h_k >= 1, h_v % h_k == 0 */
    int32_t d_k, d_v;      /* head dims; this build: 64 or 128 each */
    int32_t qkv_dtype;     /* gdn_dtype of q, k, v, conv weight, bias, conv states */
    int32_t out_dtype;     /* gdn_dtype of o */
    float scale;           /* multiplier of S q; 0 => d_k^{-1/2} */
    int32_t qk_l2norm;     /* 1 => L2-normalise q and k per head; 0 => no */
    float l2_eps;          /* eps of the L2 norm; 0 => 1e-6 */
    int32_t conv_width;    /* 0 => no conv prologue (no SiLU); 4 => conv + SiLU */
    int32_t beta_logits;   /* 0 => beta is the write strength as given; 1 => beta
                            * holds the raw gate b and the kernels use
                            * sigmoid(b) = 1 / (1 + e^{-b}) in fp32, the fused
                            * sigmoid gating of the decode update ("[Feature] Add
                            * batch invariance support to GDN_ATTN backend",
                            * PR description, section "Solution": decode goes
                            * through fused_sigmoid_gating_delta_rule_update) */
    int32_t segment_chunks; /* prefill only.  0 => one dependent chain per
                            * sequence.  > 0 => segment split: a sequence of
                            * nch > segment_chunks 64-token chunks runs as
                            * S = ceil(nch / segment_chunks) segments of
                            * ceil(nch / S) chunks, in parallel; each segment
                            * after the first starts from zero state, beside
                            * d_k identity columns that give its d_k x d_k
                            * transition and its outputs' dependence on the
                            * start state; the start states are then chained
                            * through the transitions and the outputs
                            * corrected by one product with them.  The split
                            * depends on each sequence's length alone, so
                            * results stay batch-invariant; they differ from
                            * the unsplit chain by rounding only.  The
                            * workspace grows by about T h_v (d_k + d_v) 4
                            * bytes plus 4 h_v d_k (d_k + d_v) bytes per
                            * segment (the analogue of the context-parallel
                            * variant of the chunked scan, "[Feature] Add
                            * batch invariance support to GDN_ATTN backend",
                            * commit messages) */
} gdn_problem;

/* Bytes of device workspace gdn_prefill_varlen needs for this problem (0 for
 * a problem the prefill rejects): the
 * chunk map (chunks before each sequence), a dispatch order of the sequences,
 * and the chunk-local terms computed in parallel over all 64-token chunks
 * (split 16-bit images of the normalised K and Q per key head, of
 * T = (I + A)^{-1} and of the decayed Q K^T per value head, and per-token
 * decay scalars), and a 16-byte descriptor per chunk slot.  That is about
 * (T + 63 N) / 64 chunk slots of 512 d_k h_k + 21504 h_v + 16 bytes each,
 * e.g. 27 KB per token for h_k = 16, h_v = 32, d_k = 128, plus the segment
 * split's buffers when segment_chunks > 0.  Depends on num_seqs,
 * total_tokens, h_k, h_v, d_k, d_v and segment_chunks; returns 0 for a NULL
 * problem or num_seqs <= 0. */
size_t gdn_prefill_workspace_bytes(const gdn_problem* p);

/*
 * Chunked prefill over packed variable-length sequences.
 *
 * The recurrence is evaluated in chunks of 64 tokens aligned to each
 * sequence start, with the recurrent state carried across chunks in fp32
 * ("[Feature] Add batch invariance support to GDN_ATTN backend", part "3.
 * The chunked delta-rule scan itself" (a): chunks are multiples of the
 * 64-token delta-rule block, state carried across chunk boundaries).
 *
 *  q, k            [T][h_k][d_k]  qkv_dtype   raw (pre-prologue) inputs
 *  v               [T][h_v][d_v]  qkv_dtype
 *  g, beta         [T][h_v]       fp32        log decay, write strength
 *  cu_seqlens      [N+1]          int32       sequence boundaries (device)
 *  conv_w          [C][4]         qkv_dtype   required when conv_width = 4
 *  conv_b          [C]            qkv_dtype   or NULL (no bias)
 *  conv_state_in   [N][C][3]      qkv_dtype   or NULL (zero history)
 *  conv_state_out  [N][C][3]      qkv_dtype   or NULL (not written); the last
 *                                 3 raw inputs of each sequence (with history
 *                                 from conv_state_in for sequences shorter
 *                                 than 3).  May be the same pointer as
 *                                 conv_state_in; no other overlap.
 *  initial_state   [N][h_v][d_k][d_v] fp32    or NULL (zero state)
 *  o               [T][h_v][d_v]  out_dtype   written for every token
 *  final_state     [N][h_v][d_k][d_v] fp32    or NULL (not written); may be
 *                                 the same pointer as initial_state.
 *  workspace       >= gdn_prefill_workspace_bytes(p) bytes, 256-byte aligned
 *
 * Length-0 sequences are allowed (final state = initial state).  o must not
 * overlap any input.  Supported: d_k, d_v in {64, 128} (any mix), bf16 or
 * fp32 inputs.  Matrix products run on the matrix cores with fp32
 * accumulation: split bf16 operands (x = hi + lo, about 16 significant bits)
 * for bf16 inputs, fp32 operands for fp32 inputs; both over the whole fp32
 * range.
 */
gdn_status gdn_prefill_varlen(const gdn_problem* p,
                              const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              const int32_t* cu_seqlens,
                              const void* conv_w, const void* conv_b,
                              const void* conv_state_in, void* conv_state_out,
                              const float* initial_state,
                              void* o, float* final_state,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * gdn_prefill_varlen with stage timing, for measurement: identical work and
 * results, plus four caller-created hipEvent_t (passed as void*) recorded on
 * `stream`: events[0] before the chunk-local kernel (norms, K K^T, T, P),
 * events[1] before the cross-chunk carry kernel, events[2] after it and
 * events[3] after the last launch.  GDN_ERR_NULL if events or any of the four
 * is NULL.  Argument errors record nothing.
 */
gdn_status gdn_prefill_varlen_timed(const gdn_problem* p,
                                    const void* q, const void* k, const void* v,
                                    const float* g, const float* beta,
                                    const int32_t* cu_seqlens,
                                    const void* conv_w, const void* conv_b,
                                    const void* conv_state_in, void* conv_state_out,
                                    const float* initial_state,
                                    void* o, float* final_state,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* events);

/*
 * Chunked prefill whose recurrent and conv states live in caller pools, as a
 * serving engine keeps them ("[Feature] Add batch invariance support to
 * GDN_ATTN backend": review comment part "3. The chunked delta-rule scan
 * itself" (a), where a continued prefill starts the scan from the stored
 * recurrent state, a new one from none, and the conv state is kept per cache
 * slot; commit messages, where the whole state pool is passed and addressed
 * by state indices, also for mixed batches).  Sequence n continues from pool
 * entry i = state_indices[n] and leaves its final states there, in place:
 *
 *  state_pool       [P][h_v][d_k][d_v] fp32  read-modify-write
 *  conv_state_pool  [P][C][3]      qkv_dtype read-modify-write (the last 3
 *                                  raw inputs, oldest first); required when
 *                                  conv_width = 4, else ignored
 *  state_indices    [N] int32 or NULL (sequence n uses entry n).  Entry -1:
 *                   the sequence starts from zero state and history, its o
 *                   rows are written and no pool entry is touched.
 *  has_initial_state [N] int32 or NULL (all 1).  0: the sequence starts from
 *                   zero state and history whatever entry i holds (a new
 *                   request); its final states still go to entry i.
 *
 * Everything else (q, k, v, g, beta, cu_seqlens, conv_w, conv_b, o,
 * workspace, stream) is as in gdn_prefill_varlen; the results equal those of
 * gdn_prefill_varlen with initial_state / conv_state_in gathered from the
 * entries, bit for bit.  A decode token is a length-1 sequence, so one call
 * can serve a mixed batch of prefills and decodes.  Indices must be in range
 * and distinct (except -1), as in gdn_decode_step; the pool sizes are not
 * passed, so o and the workspace are only checked not to start at a pool.
 */
gdn_status gdn_prefill_varlen_pooled(const gdn_problem* p,
                                     const void* q, const void* k, const void* v,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens,
                                     const void* conv_w, const void* conv_b,
                                     void* conv_state_pool, float* state_pool,
                                     const int32_t* state_indices,
                                     const int32_t* has_initial_state,
                                     void* o, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * gdn_prefill_varlen for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, bit for bit, with no
 * workspace argument.  The workspace lives in a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; its address is looked up once per device, at
 * the first call with that device current.  Problems whose
 * gdn_prefill_workspace_bytes() exceeds GDN_NOALLOC_SCRATCH_BYTES return
 * GDN_ERR_SCRATCH (e.g. more than about 4,700 tokens in one call at
 * h_k = 16, h_v = 32, d = 128).  The call allocates and frees nothing.
 * Calls on one GPU share its array: calls that overlap in time on one GPU
 * (different streams, or different host threads) race and must be ordered by
 * the caller.  Every byte a call reads from the array it has written earlier
 * in the same call, so no clearing is needed between calls.  `stream` must
 * belong to the current device (GDN_ERR_UNSUPPORTED otherwise).  Other
 * arguments, errors and conventions as in gdn_prefill_varlen.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_prefill_varlen_noalloc(const gdn_problem* p,
                                      const void* q, const void* k, const void* v,
                                      const float* g, const float* beta,
                                      const int32_t* cu_seqlens,
                                      const void* conv_w, const void* conv_b,
                                      const void* conv_state_in, void* conv_state_out,
                                      const float* initial_state,
                                      void* o, float* final_state,
                                      void* stream);

/*
 * One decode step: one new token for each of N slots, updating a pooled
 * state in place ("[Feature] Add batch invariance support to GDN_ATTN
 * backend", commit messages: the decode update runs over the state pool
 * addressed by ssm_state_indices, in place).
 *
 *  q, k             [N][h_k][d_k]  qkv_dtype
 *  v                [N][h_v][d_v]  qkv_dtype
 *  g, beta          [N][h_v]       fp32
 *  conv_w, conv_b   as in prefill; conv_w required when conv_width = 4
 *  conv_state_pool  [P][C][3]      qkv_dtype  read-modify-write (shifted to
 *                                  hold the newest 3 raw inputs); required
 *                                  when conv_width = 4, else ignored
 *  state_pool       [P][h_v][d_k][d_v] fp32   read-modify-write
 *  state_indices    [N] int32 or NULL (slot n uses pool entry n); entry -1
 *                   skips the slot (its o row and pool entries untouched)
 *  o                [N][h_v][d_v]  out_dtype
 *
 * p->total_tokens must equal p->num_seqs.  Each slot is computed alone, so
 * results do not depend on N or on the other slots.  Supported: d_k, d_v in
 * {64, 128}, any qkv dtype.  The pools must not overlap q, k, v, g, beta,
 * conv_w, conv_b, state_indices or o (GDN_ERR_ALIAS when an input or o
 * covers a pool's first byte; other overlaps are not detected).
 */
gdn_status gdn_decode_step(const gdn_problem* p,
                           const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           const void* conv_w, const void* conv_b, void* conv_state_pool,
                           float* state_pool, const int32_t* state_indices,
                           void* o, void* stream);

/*
 * Multi-token (speculative) decode: m = tokens_per_slot new tokens for each of
 * N slots, applied in order in one call ("[Feature] Add batch invariance
 * support to GDN_ATTN backend", commit messages: decode runs as separate spec
 * and non-spec paths over the state pool addressed by state indices).  The
 * state after every token can be kept, so a caller that accepts only the
 * first a tokens of a slot resumes from the state after token a - 1.
 *
 *  q, k             [N * m][h_k][d_k]  qkv_dtype  slot-major: row n * m + j
 *                                                 is token j of slot n
 *  v                [N * m][h_v][d_v]  qkv_dtype
 *  g, beta          [N * m][h_v]       fp32
 *  conv_w, conv_b, conv_state_pool     as in gdn_decode_step
 *  state_pool       [P][h_v][d_k][d_v] fp32      read-modify-write
 *  state_indices    [N][m] int32, or NULL.  With indices, slot n reads its
 *                   recurrent state and conv history from entry
 *                   idx[n][a_n - 1] (a_n = num_accepted[n]) and writes the
 *                   state and conv history after token j to entry idx[n][j]
 *                   (not written when idx[n][j] = -1; the read entry may be
 *                   one of them).  idx[n][a_n - 1] = -1 skips the slot: its o
 *                   rows and every pool entry stay untouched.  NULL: slot n
 *                   reads entry n and writes the state after its last token
 *                   back to entry n.
 *  num_accepted     [N] int32 in 1..m, or NULL (all 1): the tokens of the
 *                   previous call the caller accepted; values outside 1..m
 *                   are clamped into it.
 *  o                [N * m][h_v][d_v]  out_dtype
 *
 * p->num_seqs = N and p->total_tokens = N * m.  tokens_per_slot: 1..8
 * (GDN_ERR_SHAPE below 1, GDN_ERR_UNSUPPORTED above 8).  Entries must be in
 * range, and distinct across slots (except -1).  Token j's results are bit
 * for bit those of j + 1 single-token gdn_decode_step calls; with m = 1 the
 * call is gdn_decode_step.  Other arguments and errors as in gdn_decode_step.
 */
gdn_status gdn_decode_multi(const gdn_problem* p, int32_t tokens_per_slot,
                            const void* q, const void* k, const void* v,
                            const float* g, const float* beta,
                            const void* conv_w, const void* conv_b, void* conv_state_pool,
                            float* state_pool, const int32_t* state_indices,
                            const int32_t* num_accepted, void* o, void* stream);

/*
 * Measurement helper (not part of the recurrence): copies `bytes` bytes from
 * src to dst on the device with a plain streaming kernel (16-byte
 * nontemporal loads and stores, `blocks` workgroups of 256 threads striding
 * over the buffers).  Timed by the benchmark as the measured HBM peak beside
 * the datasheet figure.  bytes a multiple of 16, pointers 16-byte aligned
 * (GDN_ERR_UNSUPPORTED), buffers disjoint (GDN_ERR_ALIAS), 1 <= blocks <= 2^20
 * (GDN_ERR_SHAPE).
 */
gdn_status gdn_stream_copy(void* dst, const void* src, size_t bytes, int32_t blocks, void* stream);

/* Static, human-readable name of a status code. */
const char* gdn_status_string(gdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
