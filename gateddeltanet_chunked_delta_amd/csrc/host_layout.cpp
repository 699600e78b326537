// Host-side sizes and support tables of the prefill and decode launches:
// plain C++ with no device code, shared by the C-ABI front end and the
// launchers.
#include "gdn_internal.h"

namespace gdn {
namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int64_t carry_blocks(int64_t chains, int64_t h_k, int64_t h_v, int64_t d_k, int64_t d_v, bool split) {
    const int64_t groups = chains * h_k, members = (h_v / h_k) * ((d_v + (split ? d_k : 0)) / kDvs);
    return (groups + 7) / 8 * 8 * members;
}

int prefill_supported(int d_k, int d_v, int qkv_dtype, int out_dtype) {
    if (out_dtype != 0 && out_dtype != 1) return 0;
    if (qkv_dtype != 0 && qkv_dtype != 1) return 0;
    return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128);
}

int decode_supported(int d_k, int d_v, int qkv_dtype, int out_dtype) {
    return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128) && (qkv_dtype == 0 || qkv_dtype == 1) &&
           (out_dtype == 0 || out_dtype == 1);
}

// Workspace: order [N] int32, chunk_base [N+1] int32, slot descriptors
// [slots] int4, K|Q images [slots][h_k] (hi and lo planes of [64][d_k]
// 16-bit units), T|P images [slots][h_v] (hi and lo planes of the lower
// blocks of two 64x64 matrices), per-token scalars [slots][h_v][4][64] fp32;
// with the segment split also chain_base [N+1], chain descriptors
// [max_chains] int4, chain order [max_chains], segment states
// [max_chains][h_v][d_k][d_v] and transitions [max_chains][h_v][d_k][d_k]
// fp32, identity-column outputs [T][h_v][d_k] and segment outputs
// [T][h_v][d_v] fp32; each region 256-byte aligned.
PrefillLayout prefill_layout(int64_t num_seqs, int64_t total_tokens, int64_t h_k, int64_t h_v, int64_t d_k,
                             int64_t d_v, int64_t segment_chunks) {
    PrefillLayout l{};
    if (num_seqs <= 0 || h_k <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return l;
    // sum_n ceil(len_n / 64) <= (T + 63 N) / 64 for any split of T tokens into N sequences
    l.slots = (total_tokens + 63 * num_seqs) / kChunk;
    size_t off = 0;
    l.order = off;
    off = align256(off + size_t(num_seqs) * sizeof(int32_t));
    l.chunk_base = off;
    off = align256(off + size_t(num_seqs + 1) * sizeof(int32_t));
    l.slot_desc = off;
    off = align256(off + size_t(l.slots) * 4 * sizeof(int32_t));
    l.kq_img = off;
    off = align256(off + size_t(l.slots) * size_t(h_k) * (4 * kChunk * size_t(d_k)) * sizeof(uint16_t));
    l.tp_img = off;
    off = align256(off + size_t(l.slots) * size_t(h_v) * (4 * kTriPieces * 8) * sizeof(uint16_t));
    l.scal_img = off;
    off = align256(off + size_t(l.slots) * size_t(h_v) * (4 * kChunk) * sizeof(float));
    l.max_chains = num_seqs;
    if (segment_chunks > 0) {
        // a sequence of nch chunks makes ceil(nch / segment_chunks) <= 1 + nch / segment_chunks chains
        l.max_chains = num_seqs + l.slots / segment_chunks;
        const size_t st = size_t(h_v) * size_t(d_k) * size_t(d_v) * sizeof(float);
        l.chain_base = off;
        off = align256(off + size_t(num_seqs + 1) * sizeof(int32_t));
        l.chain_desc = off;
        off = align256(off + size_t(l.max_chains) * 4 * sizeof(int32_t));
        l.chain_order = off;
        off = align256(off + size_t(l.max_chains) * sizeof(int32_t));
        l.seg_state = off;
        off = align256(off + size_t(l.max_chains) * st);
        l.seg_trans = off;
        off = align256(off + size_t(l.max_chains) * size_t(h_v) * size_t(d_k) * size_t(d_k) * sizeof(float));
        l.seg_y = off;
        off = align256(off + size_t(total_tokens) * size_t(h_v) * size_t(d_k) * sizeof(float));
        l.seg_oloc = off;
        off = align256(off + size_t(total_tokens) * size_t(h_v) * size_t(d_v) * sizeof(float));
    }
    l.bytes = off;
    l.prep_blocks = l.slots * h_k;
    l.carry_blocks = carry_blocks(l.max_chains, h_k, h_v, d_k, d_v, segment_chunks > 0);
    return l;
}

}  // namespace gdn
