// C ABI front end: argument validation (before any HIP call) and launch.
#include <math.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes > 0 ? bytes : 0)};
}

bool overlaps(Range a, Range b) {
    if (a.lo == 0 || b.lo == 0 || a.hi == a.lo || b.hi == b.lo) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t elem_bytes(int32_t dt) { return dt == GDN_BF16 ? 2 : 4; }

// Common checks on the problem description.
gdn_status check_problem(const gdn_problem* p) {
    if (!p) return GDN_ERR_NULL;
    if (p->qkv_dtype != GDN_F32 && p->qkv_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (p->out_dtype != GDN_F32 && p->out_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (p->num_seqs < 0 || p->total_tokens < 0) return GDN_ERR_SHAPE;
    if (p->h_k < 1 || p->h_v < 1 || p->h_v % p->h_k != 0) return GDN_ERR_SHAPE;
    if (p->d_k < 1 || p->d_v < 1) return GDN_ERR_SHAPE;
    if (p->conv_width != 0 && p->conv_width != 4) return GDN_ERR_UNSUPPORTED;
    if (p->qk_l2norm != 0 && p->qk_l2norm != 1) return GDN_ERR_SHAPE;
    if (p->beta_logits != 0 && p->beta_logits != 1) return GDN_ERR_SHAPE;
    if (!isfinite(p->scale) || !isfinite(p->l2_eps) || p->l2_eps < 0.0f) return GDN_ERR_SHAPE;
    if (p->segment_chunks < 0) return GDN_ERR_SHAPE;
    // keep every element offset well inside int64 and grid sizes inside 2^31
    if (p->total_tokens > (int64_t(1) << 31) || p->num_seqs > (1 << 24) || p->h_v > 4096 ||
        p->h_k > 4096 || p->d_k > 4096 || p->d_v > 4096)
        return GDN_ERR_SHAPE;
    return GDN_OK;
}

float eff_scale(const gdn_problem* p) { return p->scale != 0.0f ? p->scale : 1.0f / sqrtf(float(p->d_k)); }
float eff_eps(const gdn_problem* p) { return p->l2_eps != 0.0f ? p->l2_eps : 1e-6f; }

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// Decode of m tokens per slot; gdn_decode_step is m = 1.
gdn_status decode(const gdn_problem* p, int32_t m, const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const void* conv_w, const void* conv_b, void* conv_state_pool,
                  float* state_pool, const int32_t* state_indices, const int32_t* num_accepted, void* o,
                  void* stream) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    const int64_t N = p->num_seqs;
    if (m < 1 || m > gdn::kDecodeMaxTokens) return m < 1 ? GDN_ERR_SHAPE : GDN_ERR_UNSUPPORTED;
    if (p->total_tokens != N * m) return GDN_ERR_SHAPE;
    if (N * p->h_k >= (int64_t(1) << 31)) return GDN_ERR_SHAPE;  // one workgroup per (slot, key head)
    if (N > 0 && (!q || !k || !v || !g || !beta || !o || !state_pool)) return GDN_ERR_NULL;
    if (p->conv_width == 4 && (!conv_w || !conv_state_pool)) return GDN_ERR_NULL;
    if (!gdn::decode_supported(p->d_k, p->d_v, p->qkv_dtype, p->out_dtype)) return GDN_ERR_UNSUPPORTED;
    if (N == 0) return GDN_OK;
    const int64_t T = N * m;
    const int64_t eb = elem_bytes(p->qkv_dtype), ob = elem_bytes(p->out_dtype);
    const int64_t nq = int64_t(p->h_k) * p->d_k, nv = int64_t(p->h_v) * p->d_v, C = 2 * nq + nv;
    if (!aligned(state_pool, 16) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(o, size_t(ob)) ||
        !aligned(q, size_t(eb)) || !aligned(k, size_t(eb)) || !aligned(v, size_t(eb)) ||
        (state_indices && !aligned(state_indices, 4)) || (num_accepted && !aligned(num_accepted, 4)))
        return GDN_ERR_UNSUPPORTED;
    // The pool sizes are not known here; check o against the per-step inputs.
    const Range ro = range_of(o, T * nv * ob);
    const Range in[] = {range_of(q, T * nq * eb), range_of(k, T * nq * eb), range_of(v, T * nv * eb),
                        range_of(g, T * p->h_v * 4), range_of(beta, T * p->h_v * 4),
                        range_of(conv_w, p->conv_width == 4 ? C * 4 * eb : 0),
                        range_of(conv_b, p->conv_width == 4 ? C * eb : 0),
                        range_of(state_indices, T * 4), range_of(num_accepted, N * 4)};
    // The pools are read and written while the inputs are read: no input may
    // reach a pool's first byte (the pool sizes are not known here).
    const Range pools[] = {range_of(state_pool, 1), range_of(conv_state_pool, 1)};
    for (const Range& r : in) {
        if (overlaps(ro, r)) return GDN_ERR_ALIAS;
        for (const Range& pr : pools)
            if (overlaps(pr, r)) return GDN_ERR_ALIAS;
    }
    if (reinterpret_cast<uintptr_t>(o) == reinterpret_cast<uintptr_t>(state_pool) ||
        (conv_state_pool && reinterpret_cast<uintptr_t>(o) == reinterpret_cast<uintptr_t>(conv_state_pool)))
        return GDN_ERR_ALIAS;

    gdn::DecodeParams prm;
    prm.q = q; prm.k = k; prm.v = v; prm.g = g; prm.beta = beta; prm.conv_w = conv_w; prm.conv_b = conv_b;
    prm.conv_state_pool = p->conv_width == 4 ? conv_state_pool : nullptr;
    prm.state_pool = state_pool; prm.state_indices = state_indices; prm.num_accepted = num_accepted; prm.o = o;
    prm.tokens = m;
    prm.num_seqs = p->num_seqs; prm.h_k = p->h_k; prm.h_v = p->h_v; prm.conv_width = p->conv_width;
    prm.beta_logits = p->beta_logits;
    prm.qk_l2norm = p->qk_l2norm; prm.l2_eps = eff_eps(p); prm.scale = eff_scale(p);
    return from_hip(gdn::launch_decode(prm, p->d_k, p->d_v, p->qkv_dtype, p->out_dtype,
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t gdn_prefill_workspace_bytes(const gdn_problem* p) {
    if (check_problem(p) != GDN_OK || p->num_seqs <= 0 ||
        !gdn::prefill_supported(p->d_k, p->d_v, p->qkv_dtype, p->out_dtype))
        return 0;
    return gdn::prefill_layout(p->num_seqs, p->total_tokens, p->h_k, p->h_v, p->d_k, p->d_v, p->segment_chunks).bytes;
}

gdn_status gdn_stream_copy(void* dst, const void* src, size_t bytes, int32_t blocks, void* stream) {
    if (bytes == 0) return GDN_OK;
    if (!dst || !src) return GDN_ERR_NULL;
    if (blocks < 1 || blocks > (1 << 20)) return GDN_ERR_SHAPE;
    if (bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16)) return GDN_ERR_UNSUPPORTED;
    if (overlaps(range_of(dst, int64_t(bytes)), range_of(src, int64_t(bytes)))) return GDN_ERR_ALIAS;
    return from_hip(gdn::launch_stream_copy(dst, src, int64_t(bytes / 16), blocks, static_cast<hipStream_t>(stream)));
}

namespace {

// Launches a validated prefill.
gdn_status launch(const gdn_problem* p, const gdn::PrefillLayout& lay, const void* q, const void* k,
                  const void* v, const float* g, const float* beta, const int32_t* cu_seqlens,
                  const void* conv_w, const void* conv_b, const void* conv_state_in, void* conv_state_out,
                  const float* initial_state, void* o, float* final_state, const int32_t* state_indices,
                  const int32_t* has_initial, void* workspace, void* stream, void* const* events) {
    gdn::PrefillParams prm;
    prm.q = q; prm.k = k; prm.v = v; prm.g = g; prm.beta = beta; prm.cu_seqlens = cu_seqlens;
    prm.conv_w = conv_w; prm.conv_b = conv_b; prm.conv_state_in = conv_state_in;
    prm.conv_state_out = conv_state_out; prm.initial_state = initial_state; prm.o = o;
    prm.final_state = final_state;
    prm.state_indices = state_indices; prm.has_initial = has_initial;
    char* ws = static_cast<char*>(workspace);
    prm.order = reinterpret_cast<int32_t*>(ws + lay.order);
    prm.chunk_base = reinterpret_cast<int32_t*>(ws + lay.chunk_base);
    prm.slot_desc = reinterpret_cast<int32_t*>(ws + lay.slot_desc);
    prm.kq_img = ws + lay.kq_img;
    prm.tp_img = ws + lay.tp_img;
    prm.scal_img = reinterpret_cast<float*>(ws + lay.scal_img);
    prm.slots = lay.slots;
    const bool split = p->segment_chunks > 0;
    prm.segment_chunks = p->segment_chunks;
    prm.chain_base = split ? reinterpret_cast<int32_t*>(ws + lay.chain_base) : nullptr;
    prm.chain_desc = split ? reinterpret_cast<int32_t*>(ws + lay.chain_desc) : nullptr;
    prm.chain_order = split ? reinterpret_cast<int32_t*>(ws + lay.chain_order) : nullptr;
    prm.seg_state = split ? reinterpret_cast<float*>(ws + lay.seg_state) : nullptr;
    prm.seg_trans = split ? reinterpret_cast<float*>(ws + lay.seg_trans) : nullptr;
    prm.seg_y = split ? reinterpret_cast<float*>(ws + lay.seg_y) : nullptr;
    prm.seg_oloc = split ? reinterpret_cast<float*>(ws + lay.seg_oloc) : nullptr;
    prm.max_chains = lay.max_chains;
    prm.num_seqs = p->num_seqs; prm.h_k = p->h_k; prm.h_v = p->h_v; prm.d_v = p->d_v;
    prm.conv_width = p->conv_width; prm.beta_logits = p->beta_logits;
    prm.qk_l2norm = p->qk_l2norm; prm.l2_eps = eff_eps(p); prm.scale = eff_scale(p);
    return from_hip(gdn::launch_prefill(prm, p->d_k, p->d_v, p->qkv_dtype, p->out_dtype,
                                        static_cast<hipStream_t>(stream), events));
}

// With noalloc the workspace arguments are ignored and the static scratch of
// the current device is used instead.
gdn_status prefill(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const int32_t* cu_seqlens, const void* conv_w, const void* conv_b,
                   const void* conv_state_in, void* conv_state_out, const float* initial_state, void* o,
                   float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                   void* const* events, bool noalloc = false) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    const int64_t T = p->total_tokens, N = p->num_seqs;
    if (N == 0 && T != 0) return GDN_ERR_SHAPE;
    if (N > 0 && !cu_seqlens) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (p->conv_width == 4 && !conv_w) return GDN_ERR_NULL;
    if (!gdn::prefill_supported(p->d_k, p->d_v, p->qkv_dtype, p->out_dtype)) return GDN_ERR_UNSUPPORTED;
    const gdn::PrefillLayout lay = gdn::prefill_layout(N, T, p->h_k, p->h_v, p->d_k, p->d_v, p->segment_chunks);
    if (N > 0 && (lay.prep_blocks >= (int64_t(1) << 31) || lay.carry_blocks >= (int64_t(1) << 31) ||
                  lay.max_chains * p->h_k >= (int64_t(1) << 31) ||
                  (p->segment_chunks > 0 && lay.slots * p->h_v * (p->d_v / 64) >= (int64_t(1) << 31))))
        return GDN_ERR_SHAPE;
    if (noalloc) {
        workspace = nullptr;  // the static scratch: no caller buffer can overlap it
        workspace_bytes = 0;
        if (N > 0 && lay.bytes > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
    } else if (N > 0 && (!workspace || workspace_bytes < lay.bytes)) {
        return GDN_ERR_WORKSPACE;
    }
    if (N == 0) return GDN_OK;

    const int64_t eb = elem_bytes(p->qkv_dtype), ob = elem_bytes(p->out_dtype);
    const int64_t nq = int64_t(p->h_k) * p->d_k, nv = int64_t(p->h_v) * p->d_v, C = 2 * nq + nv;
    const int64_t state_bytes = N * p->h_v * int64_t(p->d_k) * p->d_v * 4;
    const void* ptrs16[] = {q, k, v, o, initial_state, final_state, workspace};
    for (const void* ptr : ptrs16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_UNSUPPORTED;
    const void* ptrs4[] = {g, beta, cu_seqlens};
    for (const void* ptr : ptrs4)
        if (ptr && !aligned(ptr, 4)) return GDN_ERR_UNSUPPORTED;
    const void* ptrse[] = {conv_w, conv_b, conv_state_in, conv_state_out};
    for (const void* ptr : ptrse)
        if (ptr && !aligned(ptr, size_t(eb))) return GDN_ERR_UNSUPPORTED;

    const Range in[] = {range_of(q, T * nq * eb), range_of(k, T * nq * eb), range_of(v, T * nv * eb),
                        range_of(g, T * p->h_v * 4), range_of(beta, T * p->h_v * 4),
                        range_of(cu_seqlens, (N + 1) * 4), range_of(conv_w, C * 4 * eb),
                        range_of(conv_b, C * eb), range_of(conv_state_in, N * C * 3 * eb),
                        range_of(initial_state, state_bytes)};
    const Range ro = range_of(o, T * nv * ob), rf = range_of(final_state, state_bytes);
    const Range rc = range_of(conv_state_out, N * C * 3 * eb), rw = range_of(workspace, int64_t(workspace_bytes));
    for (const Range& r : in) {
        if (overlaps(ro, r) || overlaps(rw, r)) return GDN_ERR_ALIAS;
        const bool same_state = r.lo == rf.lo && initial_state == final_state && r.hi == rf.hi;
        if (!same_state && overlaps(rf, r)) return GDN_ERR_ALIAS;
        const bool same_conv = r.lo == rc.lo && conv_state_in == conv_state_out && r.hi == rc.hi;
        if (!same_conv && overlaps(rc, r)) return GDN_ERR_ALIAS;
    }
    if (overlaps(ro, rf) || overlaps(ro, rc) || overlaps(ro, rw) || overlaps(rf, rc) || overlaps(rf, rw) ||
        overlaps(rc, rw))
        return GDN_ERR_ALIAS;

    if (noalloc) {
        // the scratch copy that is used is the current device's: the stream
        // must run on it
        int cur = -1;
        hipDevice_t sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess ||
            hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return GDN_ERR_HIP;
        if (sdev != cur) return GDN_ERR_UNSUPPORTED;
        size_t bytes = 0;
        if (gdn::noalloc_scratch(&workspace, &bytes) != hipSuccess) return GDN_ERR_HIP;
        if (bytes < lay.bytes) return GDN_ERR_SCRATCH;
    }
    return launch(p, lay, q, k, v, g, beta, cu_seqlens, conv_w, conv_b, conv_state_in, conv_state_out,
                  initial_state, o, final_state, nullptr, nullptr, workspace, stream, events);
}

gdn_status prefill_pooled(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, const void* conv_w, const void* conv_b,
                          void* conv_state_pool, float* state_pool, const int32_t* state_indices,
                          const int32_t* has_initial, void* o, void* workspace, size_t workspace_bytes,
                          void* stream) {
    gdn_status st = check_problem(p);
    if (st != GDN_OK) return st;
    const int64_t T = p->total_tokens, N = p->num_seqs;
    if (N == 0 && T != 0) return GDN_ERR_SHAPE;
    if (N > 0 && (!cu_seqlens || !state_pool)) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (p->conv_width == 4 && (!conv_w || !conv_state_pool)) return GDN_ERR_NULL;
    if (!gdn::prefill_supported(p->d_k, p->d_v, p->qkv_dtype, p->out_dtype)) return GDN_ERR_UNSUPPORTED;
    const gdn::PrefillLayout lay = gdn::prefill_layout(N, T, p->h_k, p->h_v, p->d_k, p->d_v, p->segment_chunks);
    if (N > 0 && (lay.prep_blocks >= (int64_t(1) << 31) || lay.carry_blocks >= (int64_t(1) << 31) ||
                  lay.max_chains * p->h_k >= (int64_t(1) << 31) ||
                  (p->segment_chunks > 0 && lay.slots * p->h_v * (p->d_v / 64) >= (int64_t(1) << 31))))
        return GDN_ERR_SHAPE;
    if (N > 0 && (!workspace || workspace_bytes < lay.bytes)) return GDN_ERR_WORKSPACE;
    if (N == 0) return GDN_OK;

    const int64_t eb = elem_bytes(p->qkv_dtype), ob = elem_bytes(p->out_dtype);
    const int64_t nq = int64_t(p->h_k) * p->d_k, nv = int64_t(p->h_v) * p->d_v, C = 2 * nq + nv;
    const void* ptrs16[] = {q, k, v, o, state_pool, workspace};
    for (const void* ptr : ptrs16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_UNSUPPORTED;
    const void* ptrs4[] = {g, beta, cu_seqlens, state_indices, has_initial};
    for (const void* ptr : ptrs4)
        if (ptr && !aligned(ptr, 4)) return GDN_ERR_UNSUPPORTED;
    const void* ptrse[] = {conv_w, conv_b, conv_state_pool};
    for (const void* ptr : ptrse)
        if (ptr && !aligned(ptr, size_t(eb))) return GDN_ERR_UNSUPPORTED;
    // The pool sizes are not known here: o and the workspace are checked
    // against the per-call inputs, and must not start at a pool.
    const Range in[] = {range_of(q, T * nq * eb), range_of(k, T * nq * eb), range_of(v, T * nv * eb),
                        range_of(g, T * p->h_v * 4), range_of(beta, T * p->h_v * 4),
                        range_of(cu_seqlens, (N + 1) * 4), range_of(conv_w, C * 4 * eb),
                        range_of(conv_b, C * eb), range_of(state_indices, N * 4), range_of(has_initial, N * 4)};
    const Range ro = range_of(o, T * nv * ob), rw = range_of(workspace, int64_t(workspace_bytes));
    for (const Range& r : in)
        if (overlaps(ro, r) || overlaps(rw, r)) return GDN_ERR_ALIAS;
    if (overlaps(ro, rw)) return GDN_ERR_ALIAS;
    const uintptr_t pools[] = {reinterpret_cast<uintptr_t>(state_pool), reinterpret_cast<uintptr_t>(conv_state_pool)};
    for (uintptr_t pool : pools)
        if (pool && (pool == reinterpret_cast<uintptr_t>(o) || pool == reinterpret_cast<uintptr_t>(workspace)))
            return GDN_ERR_ALIAS;
    if (conv_state_pool && reinterpret_cast<uintptr_t>(conv_state_pool) == reinterpret_cast<uintptr_t>(state_pool))
        return GDN_ERR_ALIAS;
    void* cpool = p->conv_width == 4 ? conv_state_pool : nullptr;
    return launch(p, lay, q, k, v, g, beta, cu_seqlens, conv_w, conv_b, cpool, cpool, state_pool, o, state_pool,
                  state_indices ? state_indices : nullptr, has_initial, workspace, stream, nullptr);
}

}  // namespace

gdn_status gdn_prefill_varlen(const gdn_problem* p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const int32_t* cu_seqlens,
                              const void* conv_w, const void* conv_b, const void* conv_state_in,
                              void* conv_state_out, const float* initial_state, void* o,
                              float* final_state, void* workspace, size_t workspace_bytes,
                              void* stream) {
    return prefill(p, q, k, v, g, beta, cu_seqlens, conv_w, conv_b, conv_state_in, conv_state_out,
                   initial_state, o, final_state, workspace, workspace_bytes, stream, nullptr);
}

gdn_status gdn_prefill_varlen_timed(const gdn_problem* p, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const int32_t* cu_seqlens,
                                    const void* conv_w, const void* conv_b, const void* conv_state_in,
                                    void* conv_state_out, const float* initial_state, void* o,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* events) {
    if (!events || !events[0] || !events[1] || !events[2] || !events[3]) return GDN_ERR_NULL;
    return prefill(p, q, k, v, g, beta, cu_seqlens, conv_w, conv_b, conv_state_in, conv_state_out,
                   initial_state, o, final_state, workspace, workspace_bytes, stream, events);
}

gdn_status gdn_prefill_varlen_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                                      const float* g, const float* beta, const int32_t* cu_seqlens,
                                      const void* conv_w, const void* conv_b, const void* conv_state_in,
                                      void* conv_state_out, const float* initial_state, void* o,
                                      float* final_state, void* stream) {
    return prefill(p, q, k, v, g, beta, cu_seqlens, conv_w, conv_b, conv_state_in, conv_state_out,
                   initial_state, o, final_state, nullptr, 0, stream, nullptr, true);
}

gdn_status gdn_prefill_varlen_pooled(const gdn_problem* p, const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const int32_t* cu_seqlens,
                                     const void* conv_w, const void* conv_b, void* conv_state_pool,
                                     float* state_pool, const int32_t* state_indices,
                                     const int32_t* has_initial_state, void* o, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return prefill_pooled(p, q, k, v, g, beta, cu_seqlens, conv_w, conv_b, conv_state_pool, state_pool,
                          state_indices, has_initial_state, o, workspace, workspace_bytes, stream);
}

gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const void* conv_w, const void* conv_b,
                           void* conv_state_pool, float* state_pool, const int32_t* state_indices, void* o,
                           void* stream) {
    return decode(p, 1, q, k, v, g, beta, conv_w, conv_b, conv_state_pool, state_pool, state_indices, nullptr, o,
                  stream);
}

gdn_status gdn_decode_multi(const gdn_problem* p, int32_t tokens_per_slot, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, const void* conv_w,
                            const void* conv_b, void* conv_state_pool, float* state_pool,
                            const int32_t* state_indices, const int32_t* num_accepted, void* o, void* stream) {
    return decode(p, tokens_per_slot, q, k, v, g, beta, conv_w, conv_b, conv_state_pool, state_pool, state_indices,
                  num_accepted, o, stream);
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "sizes inconsistent or out of range";
        case GDN_ERR_DTYPE: return "unknown dtype";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration or misaligned pointer";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "HIP kernel launch failed";
        case GDN_ERR_ALIAS: return "an output overlaps a buffer it must not";
        case GDN_ERR_SCRATCH: return "problem needs more workspace than the static scratch of the no-alloc entry point";
    }
    return "unknown status";
}

}  // extern "C"
