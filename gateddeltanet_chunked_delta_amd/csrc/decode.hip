// Decode of the gated delta rule on gfx950: m >= 1 new tokens for each of N
// slots of a pooled state, in order.
//
// One workgroup per (slot, key head) handles the value heads that share that
// key head.  For each of them it streams the fp32 state tile H = S^T
// (d_k x d_v, d_v contiguous) from HBM once, applies the m tokens with the
// tile in registers, and writes it back after every token that has an entry
// to go to:
//   p = H^T k,  s = H^T q            (one pass over H)
//   delta = beta (v - e^g p)
//   o = scale (e^g s + delta (k . q))   = scale S_t q  without a second pass
//   H <- e^g H + k delta^T
// ("[Feature] Add batch invariance support to GDN_ATTN backend", commit
// messages: the decode update runs in place over the state pool addressed by
// state indices, with separate spec and non-spec decode paths; the rule
// itself is "Qwen3.5-27B GPTQ Garbage Inference -- Root Cause Analysis",
// section "Why abliteration failed on Qwen3.5", item 3.)
// With m > 1 (speculative tokens) the state after token j goes to pool entry
// idx[n][j], so a caller that accepts only the first a tokens continues from
// entry idx[n][a - 1]; the next call reads its state from
// idx[n][accepted[n] - 1].  The conv history is handled the same way.
// Every q|k|v channel's conv history is read and shifted by the one thread
// that owns the channel, so the pooled conv state is updated in the same
// launch without a race.  Reductions over d_k run in a fixed order inside the
// workgroup, the same for every token, so each slot is computed identically
// whatever the batch, and m tokens in one call give bit for bit the results
// of m single-token calls.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// 512 threads per workgroup: 8 float4 of a d=128 state tile per thread and
// head (256 threads with 16 measured 4% slower).  State accesses are
// nontemporal: the pool is streamed once per step and should not displace
// other data in the caches.
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

// Every multiply-add below is an explicit fmaf (or an explicit separate
// product), so the rounding does not depend on which products the compiler
// would contract: both kernel variants compute each token identically.

// Fixed-pattern butterfly sum over a full wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One channel's conv(4) + SiLU over the m <= KMAX new inputs of a slot, in
// order.  The 3-input history is read from entry `rslot` of the conv pool;
// the history after token j (the newest 3 raw inputs) is written to entry
// wslot(j) when that is >= 0.  The history is held in registers, so any
// entry may be both read and written.  out[j * stride] receives token j.
// The inputs, the taps and the pool do not overlap (the caller checks that o
// and the inputs are apart; the pool is neither), so the compiler may issue
// the next token's input load ahead of this token's history stores.
template <typename TIn, typename WSlot>
__device__ __forceinline__ void conv_tokens(const TIn* __restrict__ cw, const TIn* __restrict__ cb,
                                            TIn* __restrict__ cs, int64_t C, int64_t ch, int rslot, WSlot wslot,
                                            const TIn* __restrict__ x, int64_t xstride, int m, float* out,
                                            int stride) {
    const TIn* hist = cs + (int64_t(rslot) * C + ch) * 3;
    TIn h0 = hist[0], h1 = hist[1], h2 = hist[2];
    const float w0 = Elem<TIn>::get(cw + ch * 4 + 0), w1 = Elem<TIn>::get(cw + ch * 4 + 1);
    const float w2 = Elem<TIn>::get(cw + ch * 4 + 2), w3 = Elem<TIn>::get(cw + ch * 4 + 3);
    const float b = cb ? Elem<TIn>::get(cb + ch) : 0.0f;
    for (int j = 0; j < m; j++) {
        const TIn xj = x[j * xstride];
        float y = b;
        y = fmaf(w0, Elem<TIn>::get(&h0), y);
        y = fmaf(w1, Elem<TIn>::get(&h1), y);
        y = fmaf(w2, Elem<TIn>::get(&h2), y);
        y = fmaf(w3, Elem<TIn>::get(&xj), y);
        h0 = h1;
        h1 = h2;
        h2 = xj;
        out[j * stride] = silu(y);
        const int ws = wslot(j);
        if (ws >= 0) {
            TIn* dst = cs + (int64_t(ws) * C + ch) * 3;
            dst[0] = h0;
            dst[1] = h1;
            dst[2] = h2;
        }
    }
}

// Minimum waves per SIMD asked of the compiler.  Two workgroups per CU (four
// waves per SIMD) need at most 128 registers; the d = 128 m-token kernel with
// bf16 inputs and outputs takes 129 unbounded and ran one workgroup per CU
// (4-token final-state call 370 -> 273 us with the bound, 4 registers
// spilled).  The others are left free: with fp32 outputs it fits in 127
// unbounded and ran 257 -> 266 us when bounded.
template <int DK, int DV, int KMAX, typename TIn, typename TOut>
constexpr int decode_min_waves() {
    return (DK == 128 && DV == 128 && KMAX > 1 && sizeof(TIn) == 2 && sizeof(TOut) == 2) ? 4 : 1;
}

// KMAX: most tokens per slot the shared buffers hold (1 for the single-token
// step, so that its LDS footprint stays minimal).
template <int DK, int DV, int KMAX, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads, (decode_min_waves<DK, DV, KMAX, TIn, TOut>())) decode_kernel(const DecodeParams p) {
    constexpr int CG = DV / 4;           // float4 column groups per row
    constexpr int RG = kThreads / CG;    // row groups
    constexpr int RPT = DK / RG;         // rows per thread
    static_assert(kThreads % CG == 0 && DK % RG == 0 && 64 % CG == 0, "decode tiling");
    static_assert(CG == 32 || CG == 16, "column sums by half- or quarter-waves (d_v = 128 or 64)");
    static_assert(2 * DK <= kThreads - KMAX && DV <= kThreads - KMAX, "one channel per thread, gate threads apart");

    // q and k of each token with channel c at (c % RG) RPT + c / RG: a thread's
    // rows rg + RG mm are contiguous
    __shared__ __attribute__((aligned(16))) float qs[KMAX][DK], ks[KMAX][DK];
    __shared__ __attribute__((aligned(16))) float vs[KMAX][DV];
    auto qk_at = [](int c) { return (c % RG) * RPT + c / RG; };
    // per-wave partial sums, double-buffered over tokens so that one barrier
    // per token suffices
    __shared__ float part[KMAX == 1 ? 1 : 2][kWaves][2][DV];
    __shared__ float scal[KMAX][4];  // |q|^2, |k|^2, raw k.q per token
    __shared__ __attribute__((aligned(16))) float fac[KMAX][4];  // 1/|q|, 1/|k|, k.q normalised
    __shared__ float gate[KMAX][2];  // e^g and beta of the current head per token

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x / p.h_k, hk = blockIdx.x % p.h_k;
    const int m = KMAX == 1 ? 1 : p.tokens;  // the single-token kernel unrolls fully
    // Pool entries: read from idx[n][accepted - 1], the state after token j
    // written to idx[n][j]; without indices entry n is read and receives the
    // state after the last token.
    const int32_t* irow = p.state_indices ? p.state_indices + int64_t(n) * m : nullptr;
    int acc = p.num_accepted ? p.num_accepted[n] : 1;
    acc = acc < 1 ? 1 : (acc > m ? m : acc);
    const int slot = irow ? irow[acc - 1] : n;
    if (slot < 0) return;
    auto wslot = [&](int j) { return irow ? irow[j] : (j == m - 1 ? n : -1); };
    const int G = p.h_v / p.h_k;
    const int64_t nq = int64_t(p.h_k) * DK, nv = int64_t(p.h_v) * DV, C = 2 * nq + nv;
    const int64_t row0 = int64_t(n) * m;  // first token row of this slot
    const TIn* cw = static_cast<const TIn*>(p.conv_w);
    const TIn* cb = static_cast<const TIn*>(p.conv_b);
    TIn* cs = static_cast<TIn*>(p.conv_state_pool);
    const bool conv = p.conv_width == 4;
    const int cg = tid % CG, rg = tid / CG;

    float* const H0 = p.state_pool + (int64_t(slot) * p.h_v + int64_t(hk) * G) * DK * DV;
    // The state loads are the bulk of the traffic: the first head's are issued
    // before anything else, each following head's as soon as the current
    // head's first reductions are done, ahead of its stores.  Over 4 rotating
    // 512 MiB pools (no cache keeps a pool between its steps) this measured
    // 185 us per step, against 190 loading each head only after the previous
    // one, and 204 with ordinary instead of nontemporal accesses.  The
    // m-token kernel loads each head's tile when it starts the head instead:
    // a second tile in registers would leave room for one workgroup per CU,
    // and its phases are long enough for two resident workgroups to overlap
    // one's loads with the other's arithmetic.
    constexpr bool kPrefetch = KMAX == 1;
    float4_t hv[RPT], hn[RPT];
    auto load_tile = [&](float4_t (&t)[RPT], const float* H) {
#pragma unroll
        for (int mm = 0; mm < RPT; mm++)
            t[mm] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(H + (rg + RG * mm) * DV) + cg);
    };
    if (kPrefetch) load_tile(hn, H0);

    for (int gi = 0; gi < G; gi++) {
        const int h = hk * G + gi;
        if (kPrefetch) {
#pragma unroll
            for (int mm = 0; mm < RPT; mm++) hv[mm] = hn[mm];
        } else {
            load_tile(hv, H0 + int64_t(gi) * DK * DV);
        }

        // ---- inputs of all m tokens: optional conv(4) + SiLU, one channel per thread ----
        if (gi == 0 && tid < 2 * DK) {
            const bool isk = tid >= DK;
            const int c = isk ? tid - DK : tid;
            const TIn* src = static_cast<const TIn*>(isk ? p.k : p.q) + row0 * nq + int64_t(hk) * DK + c;
            float* dst = isk ? &ks[0][qk_at(c)] : &qs[0][qk_at(c)];
            if (conv) {
                const int64_t ch = (isk ? nq : 0) + int64_t(hk) * DK + c;
                conv_tokens<TIn>(cw, cb, cs, C, ch, slot, wslot, src, nq, m, dst, DK);
            } else {
                for (int j = 0; j < m; j++) dst[j * DK] = Elem<TIn>::get(src + j * nq);
            }
        }
        // the gates of this head, off the per-token critical path
        if (tid >= kThreads - KMAX && tid - (kThreads - KMAX) < m) {
            const int64_t tok = row0 + (tid - (kThreads - KMAX));
            gate[tid - (kThreads - KMAX)][0] = expf(p.g[tok * p.h_v + h]);
            gate[tid - (kThreads - KMAX)][1] = beta_of(p.beta[tok * p.h_v + h], p.beta_logits != 0);
        }
        if (tid < DV) {
            const TIn* src = static_cast<const TIn*>(p.v) + row0 * nv + int64_t(h) * DV + tid;
            if (conv) {
                const int64_t ch = 2 * nq + int64_t(h) * DV + tid;
                conv_tokens<TIn>(cw, cb, cs, C, ch, slot, wslot, src, nv, m, &vs[0][tid], DV);
            } else {
                for (int j = 0; j < m; j++) vs[j][tid] = Elem<TIn>::get(src + j * nv);
            }
        }
        __syncthreads();
        // ---- norms and k.q of every token (one wave per quantity; fixed order), once per key head ----
        if (gi == 0) {
            for (int it = wave; it < 3 * m; it += kWaves) {
                const int j = it / 3, w = it % 3;
                float a = 0.0f;
#pragma unroll
                for (int mm = 0; mm < DK / 64; mm++) {
                    const int i = lane + 64 * mm;
                    const int at = qk_at(i);
                    const float x = w == 1 ? ks[j][at] : qs[j][at], y = w == 0 ? qs[j][at] : ks[j][at];
                    a = fmaf(x, y, a);
                }
                a = wave_sum(a);
                if (lane == 0) scal[j][w] = a;
            }
            __syncthreads();
            if (tid < m) {
                const float rq = p.qk_l2norm ? 1.0f / sqrtf(scal[tid][0] + p.l2_eps) : 1.0f;
                const float rk = p.qk_l2norm ? 1.0f / sqrtf(scal[tid][1] + p.l2_eps) : 1.0f;
                fac[tid][0] = rq;
                fac[tid][1] = rk;
                fac[tid][2] = scal[tid][2] * rq * rk;
            }
            __syncthreads();
        }

        for (int j = 0; j < m; j++) {
            const float4 f4 = *reinterpret_cast<const float4*>(fac[j]);
            const float rq = f4.x, rk = f4.y, kq = f4.z;
            // ---- p = H^T k, s = H^T q over this thread's rows ----
            float pk[4] = {0.0f, 0.0f, 0.0f, 0.0f}, pq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            float kr[RPT], qr[RPT];
            if constexpr (RPT % 4 == 0) {
#pragma unroll
                for (int mm = 0; mm < RPT; mm += 4) {
                    const float4 k4 = *reinterpret_cast<const float4*>(&ks[j][rg * RPT + mm]);
                    const float4 q4 = *reinterpret_cast<const float4*>(&qs[j][rg * RPT + mm]);
                    kr[mm] = k4.x * rk, kr[mm + 1] = k4.y * rk, kr[mm + 2] = k4.z * rk, kr[mm + 3] = k4.w * rk;
                    qr[mm] = q4.x * rq, qr[mm + 1] = q4.y * rq, qr[mm + 2] = q4.z * rq, qr[mm + 3] = q4.w * rq;
                }
            } else {
#pragma unroll
                for (int mm = 0; mm < RPT; mm++) {
                    kr[mm] = ks[j][rg * RPT + mm] * rk;
                    qr[mm] = qs[j][rg * RPT + mm] * rq;
                }
            }
#pragma unroll
            for (int mm = 0; mm < RPT; mm++) {
                const float kk = kr[mm], qq = qr[mm];
                const float h4[4] = {hv[mm][0], hv[mm][1], hv[mm][2], hv[mm][3]};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    pk[e] = fmaf(h4[e], kk, pk[e]);
                    pq[e] = fmaf(h4[e], qq, pq[e]);
                }
            }
            // row groups inside a wave: lanes that differ in the bits above CG
#pragma unroll
            for (int o = CG; o < 64; o <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    pk[e] += __shfl_xor(pk[e], o);
                    pq[e] += __shfl_xor(pq[e], o);
                }
            }
            float(*pt)[2][DV] = part[KMAX == 1 ? 0 : (j & 1)];
            if (lane < CG) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    pt[wave][0][4 * cg + e] = pk[e];
                    pt[wave][1][4 * cg + e] = pq[e];
                }
            }
            __syncthreads();
            if (kPrefetch && gi + 1 < G) load_tile(hn, H0 + int64_t(gi + 1) * DK * DV);
            const int64_t tok = row0 + j;
            const float decay = gate[j][0], b = gate[j][1];
            // The waves' partials of this lane's 4 columns, summed in wave
            // order (d_v = 64: waves 0-3 and 4-7 summed apart, then added).
            // With 32 column groups the two half-waves hold the same columns:
            // the lower half sums p, the upper s, and they swap.
            float skv[4], sqv[4];
            if constexpr (CG == 32) {
                const int qn = lane >> 5;
                float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int w = 0; w < kWaves; w++) {
                    const float4 v4 = *reinterpret_cast<const float4*>(&pt[w][qn][4 * cg]);
                    a[0] += v4.x;
                    a[1] += v4.y;
                    a[2] += v4.z;
                    a[3] += v4.w;
                }
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[e]), __float_as_uint(a[e]), false, false);
                    const float o = __uint_as_float(qn ? sw[0] : sw[1]);
                    skv[e] = qn ? o : a[e];
                    sqv[e] = qn ? a[e] : o;
                }
            } else if constexpr (CG == 16) {
                // Four quarter-waves over the same columns: quarter qn sums
                // quantity qn & 1 (p, s) over waves 4 (qn >> 1) .. 4 (qn >> 1) + 3;
                // the two wave halves are added across lanes l, l ^ 32 (the
                // first half's sum first), then p and s swap across l, l ^ 16.
                const int qn = lane >> 4, which = qn & 1, wlo = 4 * (qn >> 1);
                float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    const float4 v4 = *reinterpret_cast<const float4*>(&pt[wlo + w][which][4 * cg]);
                    a[0] += v4.x;
                    a[1] += v4.y;
                    a[2] += v4.z;
                    a[3] += v4.w;
                }
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[e]), __float_as_uint(a[e]), false, false);
                    const float o = __uint_as_float((qn >> 1) ? sw[0] : sw[1]);
                    const float t = (qn >> 1) ? o + a[e] : a[e] + o;
                    const auto sw2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
                    const float o2 = __uint_as_float(which ? sw2[0] : sw2[1]);
                    skv[e] = which ? o2 : t;
                    sqv[e] = which ? t : o2;
                }
            }
            const float4 v4 = *reinterpret_cast<const float4*>(&vs[j][4 * cg]);
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
            float dlt[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int c = 4 * cg + e;
                const float sk = skv[e], sq = sqv[e];
                dlt[e] = b * fmaf(-decay, sk, vv[e]);
                if (rg == 0) {
                    TOut* op = static_cast<TOut*>(p.o) + (tok * p.h_v + h) * DV + c;
                    Elem<TOut>::put(op, p.scale * fmaf(decay, sq, dlt[e] * kq));
                }
            }
            // ---- H <- e^g H + k delta^T, written to the token's entry ----
            const int ws = wslot(j);
            float* Hw = p.state_pool + (int64_t(ws) * p.h_v + h) * DK * DV;
#pragma unroll
            for (int mm = 0; mm < RPT; mm++) {
                const int i = rg + RG * mm;
                const float kk = kr[mm];
#pragma unroll
                for (int e = 0; e < 4; e++) hv[mm][e] = fmaf(kk, dlt[e], decay * hv[mm][e]);
                if (ws >= 0) __builtin_nontemporal_store(hv[mm], reinterpret_cast<float4_t*>(Hw + i * DV) + cg);
            }
            // A wave writes token j + 2's partial sums into this token's
            // buffer only after every wave has passed token j + 1's barrier,
            // i.e. has finished reading this one; vs, qs and ks are rewritten
            // by the next head.
            if (j == m - 1) __syncthreads();
        }
    }
}

template <int DK, int DV, typename TIn, typename TOut>
hipError_t run(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid(unsigned(int64_t(p.num_seqs) * p.h_k)), block(kThreads);
    if (p.tokens == 1)
        decode_kernel<DK, DV, 1, TIn, TOut><<<grid, block, 0, stream>>>(p);
    else
        decode_kernel<DK, DV, kDecodeMaxTokens, TIn, TOut><<<grid, block, 0, stream>>>(p);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t run_dims(const DecodeParams& p, int d_k, int d_v, hipStream_t stream) {
    if (d_k == 128 && d_v == 128) return run<128, 128, TIn, TOut>(p, stream);
    if (d_k == 128 && d_v == 64) return run<128, 64, TIn, TOut>(p, stream);
    if (d_k == 64 && d_v == 128) return run<64, 128, TIn, TOut>(p, stream);
    if (d_k == 64 && d_v == 64) return run<64, 64, TIn, TOut>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype,
                         hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    if (p.tokens < 1 || p.tokens > kDecodeMaxTokens) return hipErrorInvalidValue;
    if (qkv_dtype == 1)
        return out_dtype == 1 ? run_dims<bf16_t, bf16_t>(p, d_k, d_v, stream) : run_dims<bf16_t, float>(p, d_k, d_v, stream);
    return out_dtype == 1 ? run_dims<float, bf16_t>(p, d_k, d_v, stream) : run_dims<float, float>(p, d_k, d_v, stream);
}

}  // namespace gdn
