// Single-token decode step of the gated delta rule on gfx950.
//
// One workgroup per (slot, key head) handles the value heads that share that
// key head.  For each of them it streams the fp32 state tile H = S^T
// (d_k x d_v, d_v contiguous) from HBM once and writes it back once:
//   p = H^T k,  s = H^T q            (one pass over H, 16-byte loads)
//   delta = beta (v - e^g p)
//   o = scale (e^g s + delta (k . q))   = scale S_t q  without a second pass
//   H <- e^g H + k delta^T
// ("[Feature] Add batch invariance support to GDN_ATTN backend", commit
// messages: the decode update runs in place over the state pool addressed by
// state indices; the rule itself is "Qwen3.5-27B GPTQ Garbage Inference --
// Root Cause Analysis", section "Why abliteration failed on Qwen3.5", item 3.)
// The conv history of every q|k|v channel is read and shifted by the one
// thread that owns the channel, so the pooled conv state is updated in the
// same launch without a race.  Reductions over d_k run in a fixed order
// inside the workgroup, so each slot is computed identically whatever the
// batch.
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

// Fixed-pattern butterfly sum over a full wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// conv(4) + SiLU of one channel's newest input x with its 3-input history,
// then the history shifted in place to hold the newest 3 inputs.
template <typename TIn>
__device__ __forceinline__ float conv_step(const TIn* cw, const TIn* cb, TIn* hist, int64_t ch, TIn xraw) {
    const TIn h0 = hist[0], h1 = hist[1], h2 = hist[2];
    float y = cb ? Elem<TIn>::get(cb + ch) : 0.0f;
    y += Elem<TIn>::get(cw + ch * 4 + 0) * Elem<TIn>::get(&h0);
    y += Elem<TIn>::get(cw + ch * 4 + 1) * Elem<TIn>::get(&h1);
    y += Elem<TIn>::get(cw + ch * 4 + 2) * Elem<TIn>::get(&h2);
    y += Elem<TIn>::get(cw + ch * 4 + 3) * Elem<TIn>::get(&xraw);
    hist[0] = h1;
    hist[1] = h2;
    hist[2] = xraw;
    return silu(y);
}

template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecodeParams p) {
    constexpr int CG = DV / 4;           // float4 column groups per row
    constexpr int RG = kThreads / CG;    // row groups
    constexpr int RPT = DK / RG;         // rows per thread
    static_assert(kThreads % CG == 0 && DK % RG == 0 && 64 % CG == 0, "decode tiling");
    static_assert(2 * DK <= kThreads && DV <= kThreads, "one channel per thread");

    __shared__ float qs[DK], ks[DK], vs[DV];
    __shared__ float part[kWaves][2][DV];
    __shared__ float scal[4];  // |q|^2, |k|^2, raw k.q

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x / p.h_k, hk = blockIdx.x % p.h_k;
    const int slot = p.state_indices ? p.state_indices[n] : n;
    if (slot < 0) return;
    const int G = p.h_v / p.h_k;
    const int64_t nq = int64_t(p.h_k) * DK, nv = int64_t(p.h_v) * DV, C = 2 * nq + nv;
    const TIn* cw = static_cast<const TIn*>(p.conv_w);
    const TIn* cb = static_cast<const TIn*>(p.conv_b);
    TIn* cs = static_cast<TIn*>(p.conv_state_pool);
    const bool conv = p.conv_width == 4;
    const int cg = tid % CG, rg = tid / CG;

    float* const H0 = p.state_pool + (int64_t(slot) * p.h_v + int64_t(hk) * G) * DK * DV;
    // The state loads are the bulk of the traffic: the first head's are issued
    // before anything else, each following head's as soon as the current
    // head's reductions are done, ahead of its stores.  Over 4 rotating
    // 512 MiB pools (no cache keeps a pool between its steps) this measured
    // 185 us per step, against 190 loading each head only after the previous
    // one, and 204 with ordinary instead of nontemporal accesses.
    float4_t hv[RPT], hn[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++)
        hn[m] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(H0 + (rg + RG * m) * DV) + cg);

    float rq = 1.0f, rk = 1.0f, kq = 0.0f;
    for (int gi = 0; gi < G; gi++) {
        const int h = hk * G + gi;
        float* H = H0 + int64_t(gi) * DK * DV;
#pragma unroll
        for (int m = 0; m < RPT; m++) hv[m] = hn[m];

        // ---- inputs: optional conv(4) + SiLU, one channel per thread ----
        if (gi == 0 && tid < 2 * DK) {
            const bool isk = tid >= DK;
            const int c = isk ? tid - DK : tid;
            const TIn* src = static_cast<const TIn*>(isk ? p.k : p.q) + int64_t(n) * nq + int64_t(hk) * DK + c;
            const int64_t ch = (isk ? nq : 0) + int64_t(hk) * DK + c;
            const float a = conv ? conv_step(cw, cb, cs + (int64_t(slot) * C + ch) * 3, ch, *src) : Elem<TIn>::get(src);
            (isk ? ks : qs)[c] = a;
        }
        if (tid < DV) {
            const TIn* src = static_cast<const TIn*>(p.v) + int64_t(n) * nv + int64_t(h) * DV + tid;
            const int64_t ch = 2 * nq + int64_t(h) * DV + tid;
            vs[tid] = conv ? conv_step(cw, cb, cs + (int64_t(slot) * C + ch) * 3, ch, *src) : Elem<TIn>::get(src);
        }
        __syncthreads();
        // ---- norms and k.q (waves 0, 1, 2; fixed order), once per key head ----
        if (gi == 0) {
            if (wave < 3) {
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m < DK / 64; m++) {
                    const int i = lane + 64 * m;
                    acc += wave == 0 ? qs[i] * qs[i] : (wave == 1 ? ks[i] * ks[i] : ks[i] * qs[i]);
                }
                acc = wave_sum(acc);
                if (lane == 0) scal[wave] = acc;
            }
            __syncthreads();
            rq = p.qk_l2norm ? 1.0f / sqrtf(scal[0] + p.l2_eps) : 1.0f;
            rk = p.qk_l2norm ? 1.0f / sqrtf(scal[1] + p.l2_eps) : 1.0f;
            kq = scal[2] * rq * rk;
        }

        // ---- p = H^T k, s = H^T q over this thread's rows ----
        float pk[4] = {0.0f, 0.0f, 0.0f, 0.0f}, pq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < RPT; m++) {
            const int i = rg + RG * m;
            const float kk = ks[i] * rk, qq = qs[i] * rq;
            const float h4[4] = {hv[m][0], hv[m][1], hv[m][2], hv[m][3]};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                pk[e] += h4[e] * kk;
                pq[e] += h4[e] * qq;
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
        if (lane < CG) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                part[wave][0][4 * cg + e] = pk[e];
                part[wave][1][4 * cg + e] = pq[e];
            }
        }
        __syncthreads();
        if (gi + 1 < G) {
#pragma unroll
            for (int m = 0; m < RPT; m++)
                hn[m] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(H + DK * DV + (rg + RG * m) * DV) + cg);
        }
        const float decay = expf(p.g[int64_t(n) * p.h_v + h]);
        const float b = beta_of(p.beta[int64_t(n) * p.h_v + h], p.beta_logits != 0);
        float dlt[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int j = 4 * cg + e;
            float sk = 0.0f, sq = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; w++) {
                sk += part[w][0][j];
                sq += part[w][1][j];
            }
            dlt[e] = b * (vs[j] - decay * sk);
            if (rg == 0) {
                TOut* op = static_cast<TOut*>(p.o) + (int64_t(n) * p.h_v + h) * DV + j;
                Elem<TOut>::put(op, p.scale * (decay * sq + dlt[e] * kq));
            }
        }
        // ---- H <- e^g H + k delta^T, written back in place ----
#pragma unroll
        for (int m = 0; m < RPT; m++) {
            const int i = rg + RG * m;
            const float kk = ks[i] * rk;
            float4_t nh;
#pragma unroll
            for (int e = 0; e < 4; e++) nh[e] = decay * hv[m][e] + kk * dlt[e];
            __builtin_nontemporal_store(nh, reinterpret_cast<float4_t*>(H + i * DV) + cg);
        }
        // vs and part are rewritten by the next value head
        __syncthreads();
    }
}

template <int DK, int DV, typename TIn, typename TOut>
hipError_t run(const DecodeParams& p, hipStream_t stream) {
    decode_kernel<DK, DV, TIn, TOut><<<dim3(unsigned(int64_t(p.num_seqs) * p.h_k)), dim3(kThreads), 0, stream>>>(p);
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

int decode_supported(int d_k, int d_v, int qkv_dtype, int out_dtype) {
    return (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128) && (qkv_dtype == 0 || qkv_dtype == 1) &&
           (out_dtype == 0 || out_dtype == 1);
}

hipError_t launch_decode(const DecodeParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype,
                         hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    if (qkv_dtype == 1)
        return out_dtype == 1 ? run_dims<bf16_t, bf16_t>(p, d_k, d_v, stream) : run_dims<bf16_t, float>(p, d_k, d_v, stream);
    return out_dtype == 1 ? run_dims<float, bf16_t>(p, d_k, d_v, stream) : run_dims<float, float>(p, d_k, d_v, stream);
}

}  // namespace gdn
