// Internal interface between the C-ABI front end (gdn_api.cpp) and the HIP
// kernels.  Not installed; the public surface is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Sizes shared by the prefill kernels and the host-side layout code.
constexpr int kChunk = 64;       // tokens per chunk, aligned to each sequence start
constexpr int kDvs = 64;         // d_v columns per carry workgroup
constexpr int kTriPieces = 320;  // 16-byte pieces of 8 columns in the lower 16x16 blocks of a 64x64 matrix

// Everything the chunked-prefill kernels need, passed by value.
struct PrefillParams {
    const void* q;              // [T][h_k][d_k]
    const void* k;              // [T][h_k][d_k]
    const void* v;              // [T][h_v][d_v]
    const float* g;             // [T][h_v]
    const float* beta;          // [T][h_v]
    const int32_t* cu_seqlens;  // [N+1]
    const void* conv_w;         // [C][4] or null
    const void* conv_b;         // [C] or null
    const void* conv_state_in;  // [N][C][3] or null
    void* conv_state_out;       // [N][C][3] or null
    const float* initial_state; // [N][h_v][d_k][d_v] or null (or a pool, see state_indices)
    void* o;                    // [T][h_v][d_v]
    float* final_state;         // [N][h_v][d_k][d_v] or null
    // Pooled states: with state_indices, sequence n's initial/final recurrent
    // state and conv history live in pool entry state_indices[n] of the
    // arrays above (-1: none, zero start and nothing written back); the
    // entry's stored contents are its initial ones unless has_initial[n] = 0.
    const int32_t* state_indices;  // [N] or null (entry n)
    const int32_t* has_initial;    // [N] or null (all 1)
    // workspace (see PrefillLayout)
    int32_t* order;             // [N] sequences, longest first
    int32_t* chunk_base;        // [N+1] chunks before each sequence
    int32_t* slot_desc;         // [slots][4] per chunk slot: sequence, first token, length, sequence start
    void* kq_img;               // [slots][h_k] K|Q split images (16-bit hi, lo planes)
    void* tp_img;               // [slots][h_v] T|P split images
    float* scal_img;            // [slots][h_v][4][64] per-token scalars
    int64_t slots;              // chunk slots: >= sum_n ceil(len_n / 64)
    // Segment split (segment_chunks > 0): a sequence of nch > segment_chunks
    // chunks runs as S = ceil(nch / segment_chunks) chains of ceil(nch / S)
    // chunks (the last one shorter); chains after the first start from zero
    // state, and chains of d_k identity columns give each segment's transition
    // and output map (see the segment kernels).  Null pointers when off.
    int32_t segment_chunks;
    int32_t* chain_base;        // [N+1] chains before each sequence
    int32_t* chain_desc;        // [max_chains][4] sequence, first chunk, chunks, segment index
    int32_t* chain_order;       // [max_chains] chains by descending length
    float* seg_state;           // [max_chains][h_v][d_k][d_v] local final state, then start state
    float* seg_trans;           // [max_chains][h_v][d_k][d_k] transition of the segment
    float* seg_y;               // [T][h_v][d_k] outputs of the identity columns (o's dependence on the start state)
    float* seg_oloc;            // [T][h_v][d_v] outputs of segments >= 1 from a zero start
    int64_t max_chains;
    int32_t num_seqs;
    int32_t h_k, h_v;
    int32_t d_v;
    int32_t conv_width;         // 0 or 4
    int32_t beta_logits;        // 1: beta holds raw gates b, use sigmoid(b)
    int32_t qk_l2norm;
    float l2_eps;
    float scale;
};

// Byte offsets of the prefill workspace regions (each 256-byte aligned) and
// the grid sizes the launches will use.
struct PrefillLayout {
    size_t order, chunk_base, slot_desc, kq_img, tp_img, scal_img;
    size_t chain_base, chain_desc, chain_order, seg_state, seg_trans, seg_y, seg_oloc;  // segment split only
    size_t bytes;
    int64_t slots, prep_blocks, carry_blocks, max_chains;
};
PrefillLayout prefill_layout(int64_t num_seqs, int64_t total_tokens, int64_t h_k, int64_t h_v, int64_t d_k,
                             int64_t d_v, int64_t segment_chunks);
// Carry workgroups of a prefill: per (chain, key head) group rounded up to a
// multiple of 8 groups (one per XCD), G value heads x d_v / kDvs slices each,
// plus G x d_k / kDvs identity slices with the segment split.  Without the
// split a chain is a sequence.
int64_t carry_blocks(int64_t chains, int64_t h_k, int64_t h_v, int64_t d_k, int64_t d_v, bool split);

// Most tokens per slot one decode call takes.
constexpr int kDecodeMaxTokens = 8;

struct DecodeParams {
    const void* q;              // [N * m][h_k][d_k], slot-major (row n * m + j = token j of slot n)
    const void* k;              // [N * m][h_k][d_k]
    const void* v;              // [N * m][h_v][d_v]
    const float* g;             // [N * m][h_v]
    const float* beta;          // [N * m][h_v]
    const void* conv_w;         // [C][4] or null
    const void* conv_b;         // [C] or null
    void* conv_state_pool;      // [P][C][3] or null
    float* state_pool;          // [P][h_v][d_k][d_v]
    const int32_t* state_indices; // [N][m] or null: read idx[n][accepted - 1], token j's state to idx[n][j]
    const int32_t* num_accepted;  // [N] in 1..m or null (all 1)
    void* o;                    // [N * m][h_v][d_v]
    int32_t tokens;             // m, tokens per slot: 1 .. kDecodeMaxTokens
    int32_t num_seqs;
    int32_t h_k, h_v;
    int32_t conv_width;
    int32_t beta_logits;        // 1: beta holds raw gates b, use sigmoid(b)
    int32_t qk_l2norm;
    float l2_eps;
    float scale;
};

// Launchers return hipSuccess or the launch error.  dtype codes follow gdn_dtype.
// events: null, or 4 hipEvent_t recorded on `stream` before the chunk-local
// kernel, before the carry kernel, after it and after the last launch.
hipError_t launch_prefill(const PrefillParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype,
                          hipStream_t stream, void* const* events);
int prefill_supported(int d_k, int d_v, int qkv_dtype, int out_dtype);

// The static workspace of gdn_prefill_varlen_noalloc on the current device:
// its device address (looked up at the first call on each device) and size.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

hipError_t launch_decode(const DecodeParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype,
                         hipStream_t stream);
int decode_supported(int d_k, int d_v, int qkv_dtype, int out_dtype);

// The measurement copy: n16 16-byte pieces from src to dst.
hipError_t launch_stream_copy(void* dst, const void* src, int64_t n16, int blocks, hipStream_t stream);

}  // namespace gdn
