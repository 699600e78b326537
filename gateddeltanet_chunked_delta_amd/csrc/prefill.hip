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
//              from the previous chunk, the conv state, or zeros); the per
//              head L2 norms of q and k are row scales, applied to the fp32
//              results of the products that read q and k.
//   A[r][s]  = beta_r e^{gam_r - gam_s} (k_r . k_s)       s <  r
//   P[r][s]  =        e^{gam_r - gam_s} (q_r . k_s)       s <= r
//   R        = diag(beta) (V - diag(e^gam) K H)
//   D        = (I + A)^{-1} R            (the per-token deltas: inverses of
//                                         the 16x16 diagonal blocks, then block
//                                         forward substitution)
//   o        = scale (diag(e^gam) Q H + P D)
//   H       <- e^{gam_last} H + K^T diag(e^{gam_last - gam}) D
// This is the delta rule S_t = e^{g_t} S_{t-1} + beta_t (v_t - e^{g_t}
// S_{t-1} k_t) k_t^T unrolled over a chunk ("Qwen3.5-27B GPTQ Garbage
// Inference -- Root Cause Analysis", section "Why abliteration failed on
// Qwen3.5", item 3).  Solving for D from the current state's residuals R
// (rather than precomputing W = (I + A)^{-1} diag(beta e^gam) K and
// U = (I + A)^{-1} diag(beta) V) skips one 64x64xd_k product per chunk, which
// suits a kernel that runs the chunks of one sequence back to back.
//
// Precision: the products with d_k-long reductions take split-fp16 operands
// (x = hi + lo 2^-11, three fp16 matrix-core steps, fp32 accumulation), about
// 22 significant bits per operand; the 16-wide block products of the
// substitution and of P D run on fp32 matrix-core steps.  A single fp16 rounding of any operand would already cost up to
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

// LDS carve-up for one workgroup.  K and Q (read by all four waves as
// matrix operands) are split-fp16 pairs (hi, lo); A, P, V and the diagonal
// inverse blocks are fp32.  Row pitches pad rows by 16 bytes so that the
// 16-byte reads of one wave spread over the banks.
template <int DK, int DVS, int VEC>
struct Smem {
    static constexpr int kPitchK = DK + 8;      // K, Q rows: [token][d_k] (fp16)
    static constexpr int kPitchF = kChunk + 4;  // A, P rows: [token][token] (fp32)
    static constexpr int kPitchV = DVS + 4;     // V rows: [token][column] (fp32)
    static constexpr int kPitchD = 20;          // diagonal inverse blocks: [4][16][kPitchD] (fp32)
    static constexpr int kRedCols = 2 * (DK / VEC);  // q|k partial sums of squares per row

    static constexpr size_t szKQ = size_t(kChunk) * kPitchK * sizeof(_Float16);
    static constexpr size_t oKhi = 0;
    static constexpr size_t oKlo = oKhi + szKQ;
    static constexpr size_t oQhi = oKlo + szKQ;
    static constexpr size_t oQlo = oQhi + szKQ;
    static constexpr size_t oA = oQlo + szKQ;
    static constexpr size_t oP = oA + size_t(kChunk) * kPitchF * sizeof(float);
    static constexpr size_t oV = oP + size_t(kChunk) * kPitchF * sizeof(float);
    static constexpr size_t oTd = oV + size_t(kChunk) * kPitchV * sizeof(float);
    static constexpr size_t oRed = oTd + size_t(4) * 16 * kPitchD * sizeof(float);  // q|k partial sums of squares
    static constexpr size_t oGam = oRed + size_t(kChunk) * kRedCols * sizeof(float);  // gam (fp64)
    // e^gam, beta, e^{gam_last-gam}, 1/|q|, 1/|k| per token, e^{gam_last}
    static constexpr size_t oScal = oGam + kChunk * sizeof(double);
    static constexpr size_t kBytes = oScal + (5 * kChunk + 4) * sizeof(float);

    static_assert(kBytes <= size_t(kLdsLimit), "LDS budget");
    static_assert(oKlo % 16 == 0 && oQhi % 16 == 0 && oQlo % 16 == 0 && oA % 16 == 0 && oP % 16 == 0 &&
                      oV % 16 == 0 && oTd % 16 == 0 && oRed % 16 == 0 &&
                      oGam % 16 == 0 && oScal % 16 == 0,
                  "16-byte aligned regions");
};

// Gram tiles of two tile-rows R0 < R1 of A B^T (A = K or Q rows, B = K rows),
// all lower tiles (R0, 0..R0) and (R1, 0..R1): R0 + R1 + 2 tiles that share
// their operand fragments, accumulated as independent split pairs.
template <int R0, int R1, int KS, int PK>
__device__ __forceinline__ void gram_two_rows(const _Float16* Ahi, const _Float16* Alo, const _Float16* Khi,
                                              const _Float16* Klo, int lr, int lg, float4_t (&acc)[R0 + R1 + 2]) {
    constexpr int NT = R0 + R1 + 2;
    float4_t hh[NT], xx[NT];
#pragma unroll
    for (int j = 0; j < NT; j++) hh[j] = xx[j] = kZero4;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const int k = 32 * ks + 8 * lg;
        const SFrag a0 = lds_sfrag(Ahi, Alo, PK, 16 * R0 + lr, k);
        const SFrag a1 = lds_sfrag(Ahi, Alo, PK, 16 * R1 + lr, k);
        SFrag b[R1 + 1];
#pragma unroll
        for (int t = 0; t <= R1; t++) b[t] = lds_sfrag(Khi, Klo, PK, 16 * t + lr, k);
#pragma unroll
        for (int t = 0; t <= R0; t++) mma3(hh[t], xx[t], a0, b[t]);
#pragma unroll
        for (int t = 0; t <= R1; t++) mma3(hh[R0 + 1 + t], xx[R0 + 1 + t], a1, b[t]);
    }
#pragma unroll
    for (int j = 0; j < NT; j++) acc[j] = combine(hh[j], xx[j]);
}

// acc += A X for a 16x16 fp32 block A (row-major at `a`, row pitch `pitch`)
// and a 16x16 X held in accumulator layout (lane l owns X[4*(l/16) + i][l%16]).
// Four fp32 K=4 matrix-core steps; in step i, lane group g = l/16 contributes
// k = 4g + i, which is exactly the element of X this lane already holds, so X
// needs no lane exchange and no precision split.
__device__ __forceinline__ void mma_blk_f32(float4_t& acc, const float* a, int pitch, const float4_t& x) {
    const int l = threadIdx.x & 63;
    const float4 av = *reinterpret_cast<const float4*>(a + (l & 15) * pitch + 4 * (l >> 4));
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, x[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, x[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, x[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, x[3], acc, 0, 0, 0);
}

// Workgroup = (sequence, value head, 64-column slice of d_v); wave w owns the
// 16 state columns [16w, 16w + 16) of the slice.  The state slice and the
// per-token residuals R and deltas D of those columns stay in registers in
// matrix-core accumulator layout; K, Q, A, P and V are shared through LDS.
template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(const PrefillParams p) {
    constexpr int DVS = 64;
    constexpr int NS = DV / DVS;
    constexpr int VEC = Elem<TIn>::kVec;
    constexpr int NGQ = DK / VEC;           // 16-byte groups per q (or k) head row
    constexpr int NG = 2 * NGQ;
    constexpr int RB = kThreads / NG;       // q|k prologue: row blocks per chunk
    constexpr int RPB = kChunk / RB;        // q|k rows per thread
    constexpr int NGV = DVS / VEC;          // 16-byte groups of a v slice row
    constexpr int VRPB = kChunk / (kThreads / NGV);  // v rows per thread
    constexpr int KT = DK / 16;             // 16-row tiles of the state column
    constexpr int KS = DK / 32;             // 32-wide steps over d_k
    static_assert(kThreads % NG == 0 && kChunk % RB == 0, "q|k prologue tiling");
    static_assert(kThreads % NGV == 0 && kChunk % (kThreads / NGV) == 0, "v prologue tiling");
    static_assert(DV % DVS == 0, "d_v slices");
    using S = Smem<DK, DVS, VEC>;
    constexpr int PK = S::kPitchK, PF = S::kPitchF, PV = S::kPitchV, PD = S::kPitchD;

    __shared__ __attribute__((aligned(16))) char smem[S::kBytes];
    _Float16* Khi = reinterpret_cast<_Float16*>(smem + S::oKhi);
    _Float16* Klo = reinterpret_cast<_Float16*>(smem + S::oKlo);
    _Float16* Qhi = reinterpret_cast<_Float16*>(smem + S::oQhi);
    _Float16* Qlo = reinterpret_cast<_Float16*>(smem + S::oQlo);
    float* Af = reinterpret_cast<float*>(smem + S::oA);
    float* Pf = reinterpret_cast<float*>(smem + S::oP);
    float* Vf = reinterpret_cast<float*>(smem + S::oV);
    float* Td = reinterpret_cast<float*>(smem + S::oTd);
    float* red = reinterpret_cast<float*>(smem + S::oRed);
    double* gam = reinterpret_cast<double*>(smem + S::oGam);
    float* eg = reinterpret_cast<float*>(smem + S::oScal);
    float* bet = eg + kChunk;
    float* dl = bet + kChunk;
    float* rq = dl + kChunk;
    float* rk = rq + kChunk;
    float* egl = rk + kChunk;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int u = blockIdx.x;
    const int slice = u % NS;
    const int h = (u / NS) % p.h_v;
    const int n = p.order[u / (NS * p.h_v)];
    const int hk = h / (p.h_v / p.h_k);
    const int wcol = 16 * wave + lr;               // this lane's column within the slice
    const int col = slice * DVS + wcol;            // ... and within d_v
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

    // Prologue assignments, fixed for the sequence: one 16-byte channel group
    // of q|k (and one of the v slice) for a block of consecutive rows of every
    // chunk.  The groups' conv taps stay in registers as raw 16-byte packs
    // (w[4 e + tap]).
    const int pg = tid % NG, prow0 = (tid / NG) * RPB;
    const int pwhich = pg / NGQ, poff = (pg % NGQ) * VEC;
    const TIn* pbase = (pwhich ? kin : qin) + hk * DK + poff;
    const int64_t pch = (pwhich ? nq : 0) + int64_t(hk) * DK + poff;
    const int vg = tid % NGV, vrow0 = (tid / NGV) * VRPB;
    const TIn* vbase = vin + int64_t(h) * DV + slice * DVS + vg * VEC;
    const int64_t vch = 2 * nq + int64_t(h) * DV + slice * DVS + vg * VEC;
    uint4 pw[4] = {}, vwp[4] = {};
    float pbias[VEC], vbias[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e++) pbias[e] = vbias[e] = 0.0f;
    if (conv) {
#pragma unroll
        for (int m = 0; m < 4; m++) {
            pw[m] = *reinterpret_cast<const uint4*>(cw + pch * 4 + m * VEC);
            vwp[m] = *reinterpret_cast<const uint4*>(cw + vch * 4 + m * VEC);
        }
        if (cb) {
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                pbias[e] = Elem<TIn>::get(cb + pch + e);
                vbias[e] = Elem<TIn>::get(cb + vch + e);
            }
        }
    }

    // conv(4) + SiLU of `rows` consecutive rows of one 16-byte channel group;
    // xr holds the raw rows from 3 before the first (zero outside the data).
    auto conv_rows = [&](const uint4* xr, const uint4 (&wp)[4], const float (&bias)[VEC], int i, float (&y)[VEC]) {
        if (conv) {
            float wv[4 * VEC], xs[4][VEC];
#pragma unroll
            for (int m = 0; m < 4; m++) Elem<TIn>::unpack16(wp[m], wv + m * VEC);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) Elem<TIn>::unpack16(xr[i + jj], xs[jj]);
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                float acc = bias[e];
#pragma unroll
                for (int jj = 0; jj < 4; jj++) acc += wv[4 * e + jj] * xs[jj][e];
                y[e] = silu(acc);
            }
        } else {
            Elem<TIn>::unpack16(xr[i + 3], y);
        }
    };

    // Raw 16-byte rows of this thread's channel groups for the chunk at cs
    // (3 rows of history from the previous chunk, the conv state or zeros;
    // rows past the chunk are zero).  All raw rows are loaded before any math.
    uint4 xr[RPB + 3], xv[VRPB + 3];
    auto load_raw = [&](int64_t cs) {
        const int Lc = int(eos - cs < kChunk ? eos - cs : kChunk);
#pragma unroll
        for (int j = 0; j < RPB + 3; j++) {
            const int row = prow0 - 3 + j;
            const int64_t tt = cs + row;
            uint4 v = {0u, 0u, 0u, 0u};
            if (row < Lc && (conv || j >= 3)) {
                if (tt >= bos) {
                    v = *reinterpret_cast<const uint4*>(pbase + tt * nq);
                } else if (csi) {
#pragma unroll
                    for (int e = 0; e < VEC; e++)
                        Elem<TIn>::set16(v, e, csi + (int64_t(n) * C + pch + e) * 3 + (3 + (tt - bos)));
                }
            }
            xr[j] = v;
        }
#pragma unroll
        for (int j = 0; j < VRPB + 3; j++) {
            const int row = vrow0 - 3 + j;
            const int64_t tt = cs + row;
            uint4 v = {0u, 0u, 0u, 0u};
            if (row < Lc && (conv || j >= 3)) {
                if (tt >= bos) {
                    v = *reinterpret_cast<const uint4*>(vbase + tt * nv);
                } else if (csi) {
#pragma unroll
                    for (int e = 0; e < VEC; e++)
                        Elem<TIn>::set16(v, e, csi + (int64_t(n) * C + vch + e) * 3 + (3 + (tt - bos)));
                }
            }
            xv[j] = v;
        }
    };
    for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
        const int L = int(eos - c0 < kChunk ? eos - c0 : kChunk);
        load_raw(c0);

        // ---- prologue: conv + SiLU.  q|k are staged un-normalised as split
        //      operands (the per-row L2 norms scale the fp32 products later);
        //      v is staged in fp32. ----
        {
#pragma unroll
            for (int i = 0; i < RPB; i++) {
                const int row = prow0 + i;
                float y[VEC];
                conv_rows(xr, pw, pbias, i, y);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < VEC; e++) {
                    if (row >= L) y[e] = 0.0f;
                    ss += y[e] * y[e];
                }
                red[row * NG + pg] = ss;
                _Float16* dhi = (pwhich ? Khi : Qhi) + row * PK + poff;
                _Float16* dlo = (pwhich ? Klo : Qlo) + row * PK + poff;
#pragma unroll
                for (int e = 0; e < VEC; e++) split1(y[e], dhi[e], dlo[e]);
            }
#pragma unroll
            for (int i = 0; i < VRPB; i++) {
                const int row = vrow0 + i;
                float y[VEC];
                conv_rows(xv, vwp, vbias, i, y);
#pragma unroll
                for (int e = 0; e < VEC; e++) Vf[row * PV + vg * VEC + e] = (row < L) ? y[e] : 0.0f;
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
        lds_barrier();

        // ---- per-row 1/|q| and 1/|k| (fixed summation order) ----
        if (tid < 2 * kChunk) {
            const int r = tid & (kChunk - 1), which = tid / kChunk;
            const float* rr = red + r * NG + which * NGQ;
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < NGQ; q++) sum += rr[q];
            (which ? rk : rq)[r] = p.qk_l2norm ? 1.0f / sqrtf(sum + p.l2_eps) : 1.0f;
        }
        lds_barrier();

        // ---- Gram tiles: A (strictly lower) and P (lower incl.), fp32.  Waves
        //      0, 1 take K K^T, waves 2, 3 take Q K^T; each wave two tile-rows
        //      ({0, 3} or {1, 2}: 5 tiles).  Tiles above the diagonal are never read. ----
        {
            const int which = wave >> 1;
            const _Float16* Ahi = which ? Qhi : Khi;
            const _Float16* Alo = which ? Qlo : Klo;
            const float* rnorm = which ? rq : rk;
            auto store_tile = [&](const float4_t& acc, int ti, int tj) {
                const int s = 16 * tj + lr, r0 = 16 * ti + 4 * lg;
                const float4 rn = *reinterpret_cast<const float4*>(rnorm + r0);
                const float4 bt = *reinterpret_cast<const float4*>(bet + r0);
                const double2 g01 = *reinterpret_cast<const double2*>(gam + r0);
                const double2 g23 = *reinterpret_cast<const double2*>(gam + r0 + 2);
                const double gs = gam[s];
                const float rks = rk[s];
                const float rnv[4] = {rn.x, rn.y, rn.z, rn.w}, btv[4] = {bt.x, bt.y, bt.z, bt.w};
                const double grv[4] = {g01.x, g01.y, g23.x, g23.y};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = r0 + e;
                    const float gram = acc[e] * rnv[e] * rks;
                    const float dec = (s <= r) ? __expf(static_cast<float>(grv[e] - gs)) : 0.0f;
                    if (which == 0) Af[r * PF + s] = (s < r) ? btv[e] * dec * gram : 0.0f;
                    else Pf[r * PF + s] = dec * gram;
                }
            };
            float4_t acc[5];
            if ((wave & 1) == 0) {
                gram_two_rows<0, 3, KS, PK>(Ahi, Alo, Khi, Klo, lr, lg, acc);
                store_tile(acc[0], 0, 0);
#pragma unroll
                for (int t = 0; t < 4; t++) store_tile(acc[1 + t], 3, t);
            } else {
                gram_two_rows<1, 2, KS, PK>(Ahi, Alo, Khi, Klo, lr, lg, acc);
                store_tile(acc[0], 1, 0);
                store_tile(acc[1], 1, 1);
#pragma unroll
                for (int t = 0; t < 3; t++) store_tile(acc[2 + t], 2, t);
            }
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
                    qh[tb][e] *= rq[r];
                    rr[tb][e] = bet[r] * (Vf[r * PV + wcol] - eg[r] * rk[r] * kh[e]);
                }
            }
        }
        lds_barrier();

        // ---- inverses of the 16x16 diagonal blocks of (I + A), by forward
        //      substitution, one column per lane (wave 0) ----
        if (wave == 0) {
            const int b = lane >> 4, c = lane & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < r; s++) acc += Af[(16 * b + r) * PF + 16 * b + s] * x[s];
                x[r] = (r < c) ? 0.0f : ((r == c) ? 1.0f : -acc);
            }
#pragma unroll
            for (int r = 0; r < 16; r++) Td[(16 * b + r) * PD + c] = x[r];
        }
        lds_barrier();

        // ---- D: block forward substitution of (I + A) D = R on this wave's
        //      column, D_b = Tbb (R_b - sum_{k<b} A_bk D_k) ----
        float4_t dacc[4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            dacc[b] = kZero4;
            mma_blk_f32(dacc[b], Td + 16 * b * PD, PD, rr[b]);
            const float4_t nd = -dacc[b];
#pragma unroll
            for (int c = b + 1; c < 4; c++) mma_blk_f32(rr[c], Af + 16 * c * PF + 16 * b, PF, nd);
        }
        // ---- o = scale (e^gam Q H + P D) ----
        {
            float4_t oacc[4];
#pragma unroll
            for (int b = 0; b < 4; b++) oacc[b] = kZero4;
#pragma unroll
            for (int k = 0; k < 4; k++)
#pragma unroll
                for (int b = k; b < 4; b++) mma_blk_f32(oacc[b], Pf + 16 * b * PF + 16 * k, PF, dacc[k]);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const float4 egv = *reinterpret_cast<const float4*>(eg + 16 * b + 4 * lg);
                const float egr[4] = {egv.x, egv.y, egv.z, egv.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 16 * b + 4 * lg + e;
                    if (r < L)
                        Elem<TOut>::put(out + ((c0 + r) * p.h_v + h) * DV + col,
                                        p.scale * (egr[e] * qh[b][e] + oacc[b][e]));
                }
            }
        }
        // ---- H <- e^{gam_last} H + K^T diag(e^{gam_last - gam} / |k|) D ----
        {
            SFrag tb2[2];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                float4_t a0, a1;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r0 = 32 * ks + 4 * lg + e, r1 = r0 + 16;
                    a0[e] = dl[r0] * rk[r0] * dacc[2 * ks][e];
                    a1[e] = dl[r1] * rk[r1] * dacc[2 * ks + 1][e];
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
        lds_barrier();
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
