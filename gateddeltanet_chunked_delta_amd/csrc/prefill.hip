// Chunked varlen prefill of the gated delta rule on gfx950.
//
// One workgroup owns one (sequence, value head, 64-column slice of d_v) and
// walks that sequence's 64-token chunks in order, keeping its slice of the
// fp32 state H (d_k x 64) in matrix-core accumulators for the whole sequence.
// Chunks are aligned to the sequence start and padded with zero rows, so a
// sequence's arithmetic never depends on the rest of the batch ("[Feature] Add
// batch invariance support to GDN_ATTN backend", commit messages: one
// cu_seqlens = [0, len] and fresh chunk indices per sequence; review part
// "3. The chunked delta-rule scan itself" (a): 64-token blocks, state carried
// across chunk boundaries).
//
// Per chunk of L <= 64 tokens, with gam_r = sum_{s<=r} g_s (chunk-local):
//   prologue   causal conv(4) + SiLU of the raw q|k|v rows (3 rows of history
//              from the previous chunk, the conv state, or zeros), then per
//              head L2 norm of q and k.
//   A[r][s]  = beta_r e^{gam_r - gam_s} (k_r . k_s)       s <  r
//   P[r][s]  =        e^{gam_r - gam_s} (q_r . k_s)       s <= r
//   T        = (I + A)^{-1}   (fp32, 16x16 diagonal blocks by substitution,
//                              off-diagonal blocks T_ij = -T_ii sum_k A_ik T_kj)
//   R        = diag(beta) (V - diag(e^gam) K H)
//   D        = T R                       (the per-token deltas)
//   o        = scale (diag(e^gam) Q H + P D)
//   H       <- e^{gam_last} H + K^T diag(e^{gam_last - gam}) D
// This is the delta rule S_t = e^{g_t} S_{t-1} + beta_t (v_t - e^{g_t}
// S_{t-1} k_t) k_t^T unrolled over a chunk ("Qwen3.5-27B GPTQ Garbage
// Inference -- Root Cause Analysis", section "Why abliteration failed on
// Qwen3.5", item 3).  Forming R from the current state and applying T to it
// (rather than precomputing W = T diag(beta e^gam) K) skips one 64x64xd_k
// product per chunk, which suits a kernel that runs the chunks of one
// sequence back to back.
//
// Precision: every matrix product takes split-fp16 operands (x = hi +
// lo 2^-11, three fp16 matrix-core steps, fp32 accumulation), about 22
// significant bits per operand.  A single fp16 rounding of any operand would already cost up to
// ~1e-2 of rms(o) in the worst element, because the outputs and states are
// sums of heavy-tailed products.  Operand magnitudes must stay below the fp16
// limit (65504); with q/k L2-normalised they are O(1).
//
// All reductions run in a fixed order inside one workgroup: no atomics and
// no batch-dependent split, so results are bit-reproducible and
// batch-invariant.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kChunk = 64;
constexpr int kThreads = 256;
constexpr int kLdsLimit = 163840;  // gfx950: 160 KiB per workgroup

// LDS carve-up for one workgroup.  Matrices shared by the four waves are held
// as split-fp16 pairs (hi, lo); row pitches pad each row by 16 bytes so that
// the 16-byte fragment reads of one wave spread over the banks.
template <int DK, int VEC>
struct Smem {
    static constexpr int kPitchK = DK + 8;      // K, Q rows: [token][d_k]
    static constexpr int kPitchT = kChunk + 8;  // A, T, P rows: [token][token]
    static constexpr int kRedCols = 2 * (DK / VEC);  // q|k partial sums of squares per row

    static constexpr size_t szKQ = size_t(kChunk) * kPitchK * sizeof(_Float16);
    static constexpr size_t szTT = size_t(kChunk) * kPitchT * sizeof(_Float16);
    static constexpr size_t oKhi = 0;
    static constexpr size_t oKlo = oKhi + szKQ;
    static constexpr size_t oQhi = oKlo + szKQ;
    static constexpr size_t oQlo = oQhi + szKQ;
    static constexpr size_t oAF = oQlo + szKQ;                 // A (fp32), later T (hi, lo)
    static constexpr size_t oTf = oAF + 2 * szTT;              // T while it is built (fp32)
    static constexpr size_t oPhi = oTf + 2 * szTT;
    static constexpr size_t oPlo = oPhi + szTT;
    static constexpr size_t oU1 = oPlo + szTT;                 // partial sums | off-diagonal blocks
    static constexpr size_t szU1a = size_t(kChunk) * kRedCols * sizeof(float);
    static constexpr size_t szU1b = size_t(3) * 256 * sizeof(float);
    static constexpr size_t szU1 = szU1a > szU1b ? szU1a : szU1b;
    static constexpr size_t oGam = oU1 + szU1;                 // gam (fp64)
    static constexpr size_t oScal = oGam + kChunk * sizeof(double);  // e^gam, beta, e^{gam_last-gam}, e^{gam_last}
    static constexpr size_t kBytes = oScal + (3 * kChunk + 4) * sizeof(float);

    static_assert(size_t(kChunk) * kPitchT * sizeof(float) == 2 * szTT, "A (fp32) and T (hi, lo) share a region");
    static_assert(kBytes <= size_t(kLdsLimit), "LDS budget");
    static_assert(oKlo % 16 == 0 && oQhi % 16 == 0 && oQlo % 16 == 0 && oAF % 16 == 0 && oTf % 16 == 0 &&
                      oPhi % 16 == 0 && oPlo % 16 == 0 && oU1 % 16 == 0 && oGam % 16 == 0 && oScal % 16 == 0,
                  "16-byte aligned regions");
};

// Lower 16x16 tiles (ti >= tj) of a 64x64 matrix, row by row.
__device__ __forceinline__ void lower_tile(int idx, int& ti, int& tj) {
    ti = (idx >= 1) + (idx >= 3) + (idx >= 6);
    tj = idx - ti * (ti + 1) / 2;
}
// Upper 16x16 tiles (ti < tj).
__device__ __forceinline__ void upper_tile(int idx, int& ti, int& tj) {
    ti = (idx >= 3) + (idx >= 5);
    tj = idx - (idx >= 3 ? (idx >= 5 ? 2 : 1) : -1);
}

// Workgroup = (sequence, value head, 64-column slice of d_v); wave w owns the
// 16 state columns [16w, 16w + 16) of the slice.  The state slice, the
// per-token residuals R and deltas D of those columns stay in registers in
// matrix-core accumulator layout; K, Q, T and P are shared through LDS.
template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(const PrefillParams p) {
    constexpr int DVS = 64;
    constexpr int NS = DV / DVS;
    constexpr int VEC = Elem<TIn>::kVec;
    constexpr int NGQ = DK / VEC;           // 16-byte groups per q (or k) head row
    constexpr int NG = 2 * NGQ;
    constexpr int IPT = kChunk * NG / kThreads;  // q|k prologue items per thread
    constexpr int KT = DK / 16;             // 16-row tiles of the state column
    constexpr int KS = DK / 32;             // 32-wide steps over d_k
    static_assert(kChunk * NG % kThreads == 0, "prologue items must split evenly");
    static_assert(DV % DVS == 0, "d_v slices");
    using S = Smem<DK, VEC>;
    constexpr int PK = S::kPitchK, PT = S::kPitchT;

    __shared__ __attribute__((aligned(16))) char smem[S::kBytes];
    _Float16* Khi = reinterpret_cast<_Float16*>(smem + S::oKhi);
    _Float16* Klo = reinterpret_cast<_Float16*>(smem + S::oKlo);
    _Float16* Qhi = reinterpret_cast<_Float16*>(smem + S::oQhi);
    _Float16* Qlo = reinterpret_cast<_Float16*>(smem + S::oQlo);
    float* Af = reinterpret_cast<float*>(smem + S::oAF);
    _Float16* Thi = reinterpret_cast<_Float16*>(smem + S::oAF);
    _Float16* Tlo = Thi + kChunk * PT;
    float* Tf = reinterpret_cast<float*>(smem + S::oTf);
    _Float16* Phi = reinterpret_cast<_Float16*>(smem + S::oPhi);
    _Float16* Plo = reinterpret_cast<_Float16*>(smem + S::oPlo);
    float* red = reinterpret_cast<float*>(smem + S::oU1);
    float* Mb = reinterpret_cast<float*>(smem + S::oU1);
    double* gam = reinterpret_cast<double*>(smem + S::oGam);
    float* eg = reinterpret_cast<float*>(smem + S::oScal);
    float* bet = eg + kChunk;
    float* dl = bet + kChunk;
    float* egl = dl + kChunk;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int u = blockIdx.x;
    const int slice = u % NS;
    const int h = (u / NS) % p.h_v;
    const int n = p.order[u / (NS * p.h_v)];
    const int hk = h / (p.h_v / p.h_k);
    const int col = slice * DVS + 16 * wave + lr;  // this lane's column of d_v
    const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
    const int64_t nq = int64_t(p.h_k) * DK, nv = int64_t(p.h_v) * DV, C = 2 * nq + nv;
    const TIn* qin = static_cast<const TIn*>(p.q);
    const TIn* kin = static_cast<const TIn*>(p.k);
    const TIn* vin = static_cast<const TIn*>(p.v);
    const TIn* cw = static_cast<const TIn*>(p.conv_w);
    const TIn* cb = static_cast<const TIn*>(p.conv_b);
    const TIn* csi = static_cast<const TIn*>(p.conv_state_in);
    TOut* out = static_cast<TOut*>(p.o);
    const bool conv = p.conv_width == 4;
    const int64_t state_base = (int64_t(n) * p.h_v + h) * DK * DV + col;

    // State column: hacc[it][e] = H[16 it + 4 lg + e][col].
    float4_t hacc[KT];
#pragma unroll
    for (int it = 0; it < KT; it++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            hacc[it][e] = p.initial_state ? p.initial_state[state_base + int64_t(16 * it + 4 * lg + e) * DV] : 0.0f;

    // Conv taps of this lane's v channel.
    const int64_t vch = 2 * nq + int64_t(h) * DV + col;
    float vw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vbias = 0.0f;
    if (conv) {
#pragma unroll
        for (int j = 0; j < 4; j++) vw[j] = Elem<TIn>::get(cw + vch * 4 + j);
        vbias = cb ? Elem<TIn>::get(cb + vch) : 0.0f;
    }

    for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
        const int L = int(eos - c0 < kChunk ? eos - c0 : kChunk);

        // ---- prologue, q|k: conv + SiLU into registers, partial sums of squares ----
        float val[IPT][VEC];
#pragma unroll
        for (int j = 0; j < IPT; j++) {
            const int item = tid + kThreads * j, r = item / NG, gi = item % NG;
            const int which = gi / NGQ, off = (gi % NGQ) * VEC;
            const TIn* base = (which ? kin : qin) + hk * DK + off;
            const int64_t ch = (which ? nq : 0) + int64_t(hk) * DK + off;
            float y[VEC];
            if (r < L) {
                const int64_t t = c0 + r;
                if (conv) {
#pragma unroll
                    for (int e = 0; e < VEC; e++) y[e] = cb ? Elem<TIn>::get(cb + ch + e) : 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 4; jj++) {
                        const int64_t tt = t - 3 + jj;
                        float x[VEC];
                        if (tt >= bos) {
                            Elem<TIn>::load16(base + tt * nq, x);
                        } else if (csi) {
#pragma unroll
                            for (int e = 0; e < VEC; e++)
                                x[e] = Elem<TIn>::get(csi + (int64_t(n) * C + ch + e) * 3 + (3 + (tt - bos)));
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; e++) x[e] = 0.0f;
                        }
#pragma unroll
                        for (int e = 0; e < VEC; e++) y[e] += Elem<TIn>::get(cw + (ch + e) * 4 + jj) * x[e];
                    }
#pragma unroll
                    for (int e = 0; e < VEC; e++) y[e] = silu(y[e]);
                } else {
                    Elem<TIn>::load16(base + t * nq, y);
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; e++) y[e] = 0.0f;
            }
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; e++) ss += y[e] * y[e];
            red[r * NG + gi] = ss;
#pragma unroll
            for (int e = 0; e < VEC; e++) val[j][e] = y[e];
        }
        // ---- prologue, v: this lane's column for tokens 16 tb + 4 lg + e ----
        float4_t vv[4];
#pragma unroll
        for (int tb = 0; tb < 4; tb++) {
            const int rb = 16 * tb + 4 * lg;
            float x[7];
#pragma unroll
            for (int j = 0; j < 7; j++) {
                const int row = rb - 3 + j;
                const int64_t tt = c0 + row;
                if (row >= L || (!conv && j < 3)) x[j] = 0.0f;
                else if (tt >= bos) x[j] = Elem<TIn>::get(vin + tt * nv + int64_t(h) * DV + col);
                else if (csi) x[j] = Elem<TIn>::get(csi + (int64_t(n) * C + vch) * 3 + (3 + (tt - bos)));
                else x[j] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 4; e++) {
                float y = x[e + 3];
                if (conv) y = silu(vbias + vw[0] * x[e] + vw[1] * x[e + 1] + vw[2] * x[e + 2] + vw[3] * x[e + 3]);
                vv[tb][e] = (rb + e < L) ? y : 0.0f;
            }
        }
        // ---- chunk-local cumulative log decay and its exponentials (wave 0) ----
        // gam reaches about -50 over a chunk; in fp32 its rounding (~4e-6
        // absolute) would become a relative error of every decay factor, which
        // the inter- and intra-chunk terms amplify.  Scan and exponentiate in fp64.
        if (wave == 0) {
            float gv = 0.0f, bv = 0.0f;
            if (lane < L) {
                gv = p.g[(c0 + lane) * p.h_v + h];
                bv = p.beta[(c0 + lane) * p.h_v + h];
            }
            double x = gv;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const double t = __shfl_up(x, o);
                if (lane >= o) x += t;
            }
            const double gl = __shfl(x, 63);
            gam[lane] = x;
            eg[lane] = static_cast<float>(exp(x));
            bet[lane] = bv;
            dl[lane] = static_cast<float>(exp(gl - x));
            if (lane == 0) egl[0] = static_cast<float>(exp(gl));
        }
        __syncthreads();

        // ---- prologue, q|k: L2 norm, stage split operands ----
#pragma unroll
        for (int j = 0; j < IPT; j++) {
            const int item = tid + kThreads * j, r = item / NG, gi = item % NG;
            const int which = gi / NGQ, off = (gi % NGQ) * VEC;
            float rn = 1.0f;
            if (p.qk_l2norm) {
                const float* rr = red + r * NG + which * NGQ;
                float s = 0.0f;
#pragma unroll
                for (int q = 0; q < NGQ; q++) s += rr[q];
                rn = 1.0f / sqrtf(s + p.l2_eps);
            }
            _Float16* dhi = (which ? Khi : Qhi) + r * PK + off;
            _Float16* dlo = (which ? Klo : Qlo) + r * PK + off;
#pragma unroll
            for (int e = 0; e < VEC; e++) split1(val[j][e] * rn, dhi[e], dlo[e]);
        }
        __syncthreads();

        // ---- Gram tiles: A (strictly lower, fp32) and P (lower incl., split) ----
        for (int job = wave; job < 20; job += 4) {
            const int which = job / 10;
            int ti, tj;
            lower_tile(job % 10, ti, tj);
            float4_t hh = kZero4, xx = kZero4;
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                mma3(hh, xx, lds_sfrag(which ? Qhi : Khi, which ? Qlo : Klo, PK, 16 * ti + lr, 32 * ks + 8 * lg),
                     lds_sfrag(Khi, Klo, PK, 16 * tj + lr, 32 * ks + 8 * lg));
            const float4_t acc = combine(hh, xx);
            const int s = 16 * tj + lr;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 16 * ti + 4 * lg + e;
                const float dec = (s <= r) ? expf(static_cast<float>(gam[r] - gam[s])) : 0.0f;
                if (which == 0) {
                    Af[r * PT + s] = (s < r) ? bet[r] * dec * acc[e] : 0.0f;
                } else {
                    const float pv = dec * acc[e];
                    split1(pv, Phi[r * PT + s], Plo[r * PT + s]);
                }
            }
        }
        for (int e = tid; e < 6 * 256; e += kThreads) {
            int ti, tj;
            upper_tile(e >> 8, ti, tj);
            const int idx = (16 * ti + ((e & 255) >> 4)) * PT + 16 * tj + (e & 15);
            Phi[idx] = _Float16(0.0f);
            Plo[idx] = _Float16(0.0f);
        }

        // ---- K H and Q H on this wave's column; R = beta (V - e^gam K H) ----
        float4_t qh[4], rr[4];
        {
            SFrag hb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                float x[8];
                acc_to_operand(hacc[2 * ks], hacc[2 * ks + 1], x);
                hb[ks] = split8(x);
            }
#pragma unroll
            for (int tb = 0; tb < 4; tb++) {
                float4_t khh = kZero4, khx = kZero4, qhh = kZero4, qhx = kZero4;
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    mma3(khh, khx, lds_sfrag(Khi, Klo, PK, 16 * tb + lr, 32 * ks + 8 * lg), hb[ks]);
                    mma3(qhh, qhx, lds_sfrag(Qhi, Qlo, PK, 16 * tb + lr, 32 * ks + 8 * lg), hb[ks]);
                }
                const float4_t kh = combine(khh, khx);
                qh[tb] = combine(qhh, qhx);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 16 * tb + 4 * lg + e;
                    rr[tb][e] = bet[r] * (vv[tb][e] - eg[r] * kh[e]);
                }
            }
        }
        __syncthreads();

        // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution ----
        if (wave == 0) {
            const int b = lane >> 4, c = lane & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < r; s++) acc += Af[(16 * b + r) * PT + 16 * b + s] * x[s];
                x[r] = (r < c) ? 0.0f : ((r == c) ? 1.0f : -acc);
            }
#pragma unroll
            for (int r = 0; r < 16; r++) Tf[(16 * b + r) * PT + 16 * b + c] = x[r];
        } else {
            for (int e = tid - 64; e < 6 * 256; e += kThreads - 64) {
                int ti, tj;
                upper_tile(e >> 8, ti, tj);
                Tf[(16 * ti + ((e & 255) >> 4)) * PT + 16 * tj + (e & 15)] = 0.0f;
            }
        }
        __syncthreads();
        // ---- off-diagonal blocks by distance: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj ----
#pragma unroll 1
        for (int d = 1; d <= 3; d++) {
            const int nb = 4 - d;
            for (int e = tid; e < nb * 256; e += kThreads) {
                const int bi = d + (e >> 8), bj = bi - d, r = (e & 255) >> 4, c = e & 15;
                float acc = 0.0f;
                for (int kb = bj; kb < bi; kb++) {
#pragma unroll
                    for (int s = 0; s < 16; s++)
                        acc += Af[(16 * bi + r) * PT + 16 * kb + s] * Tf[(16 * kb + s) * PT + 16 * bj + c];
                }
                Mb[e] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nb * 256; e += kThreads) {
                const int bi = d + (e >> 8), bj = bi - d, r = (e & 255) >> 4, c = e & 15;
                const float* m = Mb + (e & ~255);
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < 16; s++) acc += Tf[(16 * bi + r) * PT + 16 * bi + s] * m[s * 16 + c];
                Tf[(16 * bi + r) * PT + 16 * bj + c] = -acc;
            }
            __syncthreads();
        }
        // T as split operand, over the (now dead) A region
        for (int e = tid; e < kChunk * kChunk; e += kThreads) {
            const int r = e >> 6, c = e & 63;
            split1(Tf[r * PT + c], Thi[r * PT + c], Tlo[r * PT + c]);
        }
        __syncthreads();

        // ---- D = T R (T lower triangular: token block tb needs K steps <= tb/2) ----
        float4_t dacc[4];
        {
            SFrag rb[2];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                float x[8];
                acc_to_operand(rr[2 * ks], rr[2 * ks + 1], x);
                rb[ks] = split8(x);
            }
#pragma unroll
            for (int tb = 0; tb < 4; tb++) {
                float4_t hh = kZero4, xx = kZero4;
#pragma unroll
                for (int ks = 0; ks <= (tb >> 1); ks++)
                    mma3(hh, xx, lds_sfrag(Thi, Tlo, PT, 16 * tb + lr, 32 * ks + 8 * lg), rb[ks]);
                dacc[tb] = combine(hh, xx);
            }
        }
        // ---- o = scale (e^gam Q H + P D) ----
        {
            SFrag db[2];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                float x[8];
                acc_to_operand(dacc[2 * ks], dacc[2 * ks + 1], x);
                db[ks] = split8(x);
            }
#pragma unroll
            for (int tb = 0; tb < 4; tb++) {
                float4_t hh = kZero4, xx = kZero4;
#pragma unroll
                for (int ks = 0; ks <= (tb >> 1); ks++)
                    mma3(hh, xx, lds_sfrag(Phi, Plo, PT, 16 * tb + lr, 32 * ks + 8 * lg), db[ks]);
                const float4_t oacc = combine(hh, xx);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 16 * tb + 4 * lg + e;
                    if (r < L)
                        Elem<TOut>::put(out + ((c0 + r) * p.h_v + h) * DV + col,
                                        p.scale * (eg[r] * qh[tb][e] + oacc[e]));
                }
            }
        }
        // ---- H <- e^{gam_last} H + K^T diag(e^{gam_last - gam}) D ----
        {
            SFrag tb2[2];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                float4_t a0, a1;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    a0[e] = dl[32 * ks + 4 * lg + e] * dacc[2 * ks][e];
                    a1[e] = dl[32 * ks + 16 + 4 * lg + e] * dacc[2 * ks + 1][e];
                }
                float x[8];
                acc_to_operand(a0, a1, x);
                tb2[ks] = split8(x);
            }
            const float decay = egl[0];
#pragma unroll
            for (int it = 0; it < KT; it++) {
                float4_t hh = hacc[it] * decay, xx = kZero4;
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
                    mma3(hh, xx, lds_sfrag_t(Khi, Klo, PK, 32 * ks + 8 * lg, 16 * it + lr), tb2[ks]);
                hacc[it] = combine(hh, xx);
            }
        }
        __syncthreads();
    }

    if (p.final_state) {
#pragma unroll
        for (int it = 0; it < KT; it++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                p.final_state[state_base + int64_t(16 * it + 4 * lg + e) * DV] = hacc[it][e];
    }
}

// Dispatch map: sequences ordered by descending chunk count (ties by index),
// so the longest dependent chains start first.  Ranks are unique, so the map
// is a permutation for any cu_seqlens contents.
__global__ void __launch_bounds__(256) order_kernel(const int32_t* __restrict__ cu, int32_t n,
                                                     int32_t* __restrict__ order) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int ci = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
    int rank = 0;
    for (int j = 0; j < n; j++) {
        const int cj = (cu[j + 1] - cu[j] + kChunk - 1) / kChunk;
        rank += (cj > ci) || (cj == ci && j < i);
    }
    order[rank] = i;
}

// Final conv state of every sequence: its last 3 raw inputs per channel,
// reaching into conv_state_in for sequences shorter than 3.  One thread per
// (sequence, channel) reads all three values before writing, so the output
// may be the input buffer itself.
template <typename TIn>
__global__ void __launch_bounds__(256) conv_state_kernel(const PrefillParams p, int dk, int dv) {
    const int64_t nq = int64_t(p.h_k) * dk, nv = int64_t(p.h_v) * dv, C = 2 * nq + nv;
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= int64_t(p.num_seqs) * C) return;
    const int64_t n = e / C, c = e % C;
    const int64_t bos = p.cu_seqlens[n], len = p.cu_seqlens[n + 1] - bos;
    const TIn* qin = static_cast<const TIn*>(p.q);
    const TIn* kin = static_cast<const TIn*>(p.k);
    const TIn* vin = static_cast<const TIn*>(p.v);
    const TIn* csi = static_cast<const TIn*>(p.conv_state_in);
    TIn* cso = static_cast<TIn*>(p.conv_state_out);
    TIn vals[3];
#pragma unroll
    for (int j = 0; j < 3; j++) {
        const int64_t pos = len - 3 + j;
        if (pos >= 0) {
            const int64_t t = bos + pos;
            vals[j] = c < nq ? qin[t * nq + c] : (c < 2 * nq ? kin[t * nq + c - nq] : vin[t * nv + c - 2 * nq]);
        } else {
            vals[j] = csi ? csi[e * 3 + 3 + pos] : TIn(0);
        }
    }
#pragma unroll
    for (int j = 0; j < 3; j++) cso[e * 3 + j] = vals[j];
}

template <int DK, int DV, typename TIn, typename TOut>
hipError_t run(const PrefillParams& p, hipStream_t stream) {
    const int64_t blocks = int64_t(p.num_seqs) * p.h_v * (DV / 64);
    prefill_kernel<DK, DV, TIn, TOut><<<dim3(unsigned(blocks)), dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t run_dtype(const PrefillParams& p, int d_k, int d_v, hipStream_t stream) {
    if (d_k == 128 && d_v == 128) return run<128, 128, TIn, TOut>(p, stream);
    if (d_k == 64 && d_v == 64) return run<64, 64, TIn, TOut>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

int prefill_supported(int d_k, int d_v, int qkv_dtype, int out_dtype) {
    if (out_dtype != 0 && out_dtype != 1) return 0;
    if (qkv_dtype != 0 && qkv_dtype != 1) return 0;
    return (d_k == 128 && d_v == 128) || (d_k == 64 && d_v == 64);
}

hipError_t launch_prefill(const PrefillParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype,
                          hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    int32_t* order = const_cast<int32_t*>(p.order);
    order_kernel<<<dim3((p.num_seqs + 255) / 256), dim3(256), 0, stream>>>(p.cu_seqlens, p.num_seqs, order);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (qkv_dtype == 1)
        err = out_dtype == 1 ? run_dtype<bf16_t, bf16_t>(p, d_k, d_v, stream) : run_dtype<bf16_t, float>(p, d_k, d_v, stream);
    else
        err = out_dtype == 1 ? run_dtype<float, bf16_t>(p, d_k, d_v, stream) : run_dtype<float, float>(p, d_k, d_v, stream);
    if (err != hipSuccess) return err;
    if (p.conv_state_out && p.conv_width == 4) {
        const int64_t total = int64_t(p.num_seqs) * (2 * int64_t(p.h_k) * d_k + int64_t(p.h_v) * d_v);
        const unsigned grid = unsigned((total + 255) / 256);
        if (qkv_dtype == 1) conv_state_kernel<bf16_t><<<dim3(grid), dim3(256), 0, stream>>>(p, d_k, d_v);
        else conv_state_kernel<float><<<dim3(grid), dim3(256), 0, stream>>>(p, d_k, d_v);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace gdn
