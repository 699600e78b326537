// Single-token decode step of the gated delta rule on gfx950.
//
// One workgroup per (slot, value head) streams that head's fp32 state tile
// H = S^T (d_k x d_v, d_v contiguous) from HBM once, and writes it back once:
//   p = H^T k,  s = H^T q            (one pass over H, 16-byte loads)
//   delta = beta (v - e^g p)
//   o = scale (e^g s + delta (k . q))   = scale S_t q  without a second pass
//   H <- e^g H + k delta^T
// ("[Feature] Add batch invariance support to GDN_ATTN backend", commit
// messages: the decode update runs in place over the state pool addressed by
// state indices; the rule itself is "Qwen3.5-27B GPTQ Garbage Inference --
// Root Cause Analysis", section "Why abliteration failed on Qwen3.5", item 3.)
// Reductions over d_k run in a fixed order inside the workgroup, so each slot
// is computed identically whatever the batch.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// 512 threads per (slot, head): 8 float4 of the state tile per thread.  With
// nontemporal loads and stores (the state is streamed once per step and should
// not displace other data in the caches) this shape reached 5.8 TB/s on an
// in-place 512 MiB read-modify-write, against 5.05 TB/s for 256 threads and
// ordinary accesses.
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

// Fixed-pattern butterfly sum over a full wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecodeParams p) {
    constexpr int CG = DV / 4;           // float4 column groups per row
    constexpr int RG = kThreads / CG;    // row groups
    constexpr int RPT = DK / RG;         // rows per thread
    static_assert(kThreads % CG == 0 && DK % RG == 0 && 64 % CG == 0, "decode tiling");

    __shared__ float qs[DK], ks[DK], vs[DV];
    __shared__ float part[kWaves][2][DV];
    __shared__ float scal[4];  // 1/||q||, 1/||k||, raw k.q

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x / p.h_v, h = blockIdx.x % p.h_v;
    const int slot = p.state_indices ? p.state_indices[n] : n;
    if (slot < 0) return;
    const int hk = h / (p.h_v / p.h_k);
    const int64_t nq = int64_t(p.h_k) * DK, nv = int64_t(p.h_v) * DV, C = 2 * nq + nv;
    const TIn* qin = static_cast<const TIn*>(p.q);
    const TIn* kin = static_cast<const TIn*>(p.k);
    const TIn* vin = static_cast<const TIn*>(p.v);
    const TIn* cw = static_cast<const TIn*>(p.conv_w);
    const TIn* cb = static_cast<const TIn*>(p.conv_b);
    const TIn* cs = static_cast<const TIn*>(p.conv_state_pool);

    float* H = p.state_pool + (int64_t(slot) * p.h_v + h) * DK * DV;
    const int cg = tid % CG, rg = tid / CG;

    // Issue the state loads first: they are the bulk of the traffic.
    float4_t hv[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++)
        hv[m] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(H + (rg + RG * m) * DV) + cg);

    // ---- inputs: optional conv(4) + SiLU with history from the conv pool ----
    for (int c = tid; c < 2 * DK + DV; c += kThreads) {
        int64_t ch;
        float x;
        if (c < DK) { ch = int64_t(hk) * DK + c; x = Elem<TIn>::get(qin + int64_t(n) * nq + hk * DK + c); }
        else if (c < 2 * DK) { ch = nq + int64_t(hk) * DK + (c - DK); x = Elem<TIn>::get(kin + int64_t(n) * nq + hk * DK + c - DK); }
        else { ch = 2 * nq + int64_t(h) * DV + (c - 2 * DK); x = Elem<TIn>::get(vin + int64_t(n) * nv + h * DV + c - 2 * DK); }
        float a = x;
        if (p.conv_width == 4) {
            const TIn* hist = cs + (int64_t(slot) * C + ch) * 3;
            float y = cb ? Elem<TIn>::get(cb + ch) : 0.0f;
            y += Elem<TIn>::get(cw + ch * 4 + 0) * Elem<TIn>::get(hist + 0);
            y += Elem<TIn>::get(cw + ch * 4 + 1) * Elem<TIn>::get(hist + 1);
            y += Elem<TIn>::get(cw + ch * 4 + 2) * Elem<TIn>::get(hist + 2);
            y += Elem<TIn>::get(cw + ch * 4 + 3) * x;
            a = silu(y);
        }
        if (c < DK) qs[c] = a;
        else if (c < 2 * DK) ks[c - DK] = a;
        else vs[c - 2 * DK] = a;
    }
    __syncthreads();
    // ---- norms and k.q (waves 0, 1, 2; fixed order) ----
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
    const float rq = p.qk_l2norm ? 1.0f / sqrtf(scal[0] + p.l2_eps) : 1.0f;
    const float rk = p.qk_l2norm ? 1.0f / sqrtf(scal[1] + p.l2_eps) : 1.0f;
    const float kq = scal[2] * rq * rk;

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
    const float decay = expf(p.g[int64_t(n) * p.h_v + h]);
    const float b = p.beta[int64_t(n) * p.h_v + h];
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
}

// Shift each used slot's conv history by one token: [s1, s2, x].  Runs after
// decode_kernel (same stream), which read the old history.
template <typename TIn>
__global__ void __launch_bounds__(256) conv_shift_kernel(const DecodeParams p, int dk, int dv) {
    const int64_t nq = int64_t(p.h_k) * dk, nv = int64_t(p.h_v) * dv, C = 2 * nq + nv;
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= int64_t(p.num_seqs) * C) return;
    const int64_t n = e / C, c = e % C;
    const int slot = p.state_indices ? p.state_indices[n] : int(n);
    if (slot < 0) return;
    const TIn* src = c < nq ? static_cast<const TIn*>(p.q) + n * nq + c
                   : (c < 2 * nq ? static_cast<const TIn*>(p.k) + n * nq + (c - nq)
                                 : static_cast<const TIn*>(p.v) + n * nv + (c - 2 * nq));
    TIn* hist = static_cast<TIn*>(p.conv_state_pool) + (int64_t(slot) * C + c) * 3;
    const TIn s1 = hist[1], s2 = hist[2], x = *src;
    hist[0] = s1;
    hist[1] = s2;
    hist[2] = x;
}

template <int DK, int DV, typename TIn, typename TOut>
hipError_t run(const DecodeParams& p, hipStream_t stream) {
    decode_kernel<DK, DV, TIn, TOut><<<dim3(unsigned(int64_t(p.num_seqs) * p.h_v)), dim3(kThreads), 0, stream>>>(p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.conv_width != 4) return err;
    const int64_t total = int64_t(p.num_seqs) * (2 * int64_t(p.h_k) * DK + int64_t(p.h_v) * DV);
    conv_shift_kernel<TIn><<<dim3(unsigned((total + 255) / 256)), dim3(256), 0, stream>>>(p, DK, DV);
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
