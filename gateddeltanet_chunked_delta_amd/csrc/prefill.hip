// Chunked varlen prefill of the gated delta rule on gfx950.
//
// The recurrence S_t = e^{g_t} S_{t-1} + beta_t (v_t - e^{g_t} S_{t-1} k_t)
// k_t^T ("Qwen3.5-27B GPTQ Garbage Inference -- Root Cause Analysis", section
// "Why abliteration failed on Qwen3.5", item 3) is evaluated in 64-token
// chunks aligned to each sequence start, zero-padded at the tail, with the
// fp32 state carried across chunks ("[Feature] Add batch invariance support
// to GDN_ATTN backend", review part "3. The chunked delta-rule scan itself"
// (a); commit messages: one cu_seqlens = [0, len] and fresh chunk indices per
// sequence).  With gam_r = sum_{s<=r} g_s inside a chunk, H = S^T and q, k
// L2-normalised:
//   A[r][s] = beta_r e^{gam_r - gam_s} (k_r . k_s)   s <  r
//   T       = (I + A)^{-1}
//   P[r][s] =        e^{gam_r - gam_s} (q_r . k_s)   s <= r
//   R       = diag(beta) (V - diag(e^gam) K H)
//   D       = T R                       (the per-token deltas)
//   o       = scale (diag(e^gam) Q H + P D)
//   H      <- e^{gam_last} H + K^T diag(e^{gam_last - gam}) D
// Everything but the last four lines is independent of H, so it runs in
// parallel over all chunks; only R, D, o and the update form the dependent
// chain over a sequence's chunks.  The launches:
//   chunk_map_kernel  chunk_base[n] = chunks before sequence n
//   slot_map_kernel   per chunk slot: its sequence, first token and length
//   order_kernel      sequences by descending chunk count (longest first)
//   (small_map_kernel: the three maps in one workgroup for up to 512
//   sequences and 65536 chunk slots)
//   prep_kernel       per (chunk, key head): conv(4) + SiLU + L2 norm of q
//                     and k; K K^T and Q K^T; then per value head of the
//                     group: the decays, T and P.  Writes split images (hi
//                     and lo planes) of K, Q, T, P and the per-token scalars to the workspace.
//   carry_kernel      per (sequence, value head, 64 columns of d_v): conv of
//                     v, then the chain above with the state slice held in
//                     matrix-core accumulators by four waves, while four
//                     helper waves stage the chunks and compute Q H, P D and
//                     the output.  The next chunk's images are loaded into
//                     registers while the current chunk computes.  At the
//                     end its helper waves write the final conv states.
// With the segment split (gdn_problem.segment_chunks > 0) a sequence longer
// than that many chunks is cut into segments carried in parallel:
//   chain_map_kernel, chain_order_kernel  the segments ("chains"), longest first
//   carry_kernel<..., true>   each segment from zero state, beside its identity
//                     chains (the d_k identity columns, v = 0), which give its
//                     transition M and the outputs' dependence Y on its start state
//   segment_combine_kernel    start states H_{s+1} = M_s H_s + F_s in order
//   segment_correct_kernel    o += Y H_s, on the matrix cores
//
// Precision: every product runs on the matrix cores with fp32 accumulation:
// split bf16 operands (x = hi + lo, three bf16 steps, about 16 significant
// bits) for bf16 inputs, fp32 operands (fp32 steps) for fp32 inputs; both
// keep the whole fp32 range.  The diagonal blocks of T
// come from an fp32 forward substitution and the off-diagonal blocks from
// fp32 matrix-core steps; the decays are scanned and exponentiated in fp64.
//
// All reductions run in a fixed order inside one workgroup, with no atomics
// and no batch-dependent split: a sequence's results are bit-identical
// whatever else shares the call.
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kLdsLimit = 163840;  // gfx950: 160 KiB per workgroup
// s_waitcnt immediate that waits for every outstanding vector memory
// operation of the wave (vmcnt = 0; expcnt and lgkmcnt left at their maxima).
constexpr int kVmcnt0 = 0x0f70;

// Workspace images, per chunk slot: [h_k] K|Q images, each a hi and a lo
// 16-bit plane (bf16 or fp16, as the operands) of [64][d_k]; [h_v] T|P images, each a hi and a lo plane of the
// 10 lower 16x16 blocks of a 64x64 matrix (TriPack); [h_v] scalar rows beta,
// e^gam, e^{gam_last - gam}, e^{gam_last}.
// A TriPack plane stores row r's columns [0, 16 (r/16 + 1)) as 16-byte
// pieces, rows in order: 320 pieces.
struct TriPack {
    static constexpr int kPieces = kTriPieces;
    // first piece of row r
    __device__ __forceinline__ static int row_start(int r) {
        const int b = r >> 4;
        return 16 * b * (b + 1) + 2 * (b + 1) * (r & 15);
    }
    // row and 8-column group of piece q
    __device__ __forceinline__ static void locate(int q, int& r, int& c8) {
        const int b = q < 32 ? 0 : (q < 96 ? 1 : (q < 192 ? 2 : 3));
        const int w = 2 * (b + 1), q0 = q - 16 * b * (b + 1);
        r = 16 * b + q0 / w;
        c8 = q0 % w;
    }
};

template <int DK>
struct Img {
    static constexpr int kKQ = 2 * 2 * kChunk * DK;            // halves per (slot, key head)
    static constexpr int kTP = 2 * 2 * TriPack::kPieces * 8;   // halves per (slot, value head)
    static constexpr int kScal = 4 * kChunk;                   // floats per (slot, value head)
};

// ---------------------------------------------------------------- prologue

// conv(4) + SiLU of rows 0..R-1 of one 16-byte channel group (xr[0 .. R+2]
// hold the raw rows from 3 before the first), with the taps and each raw row
// unpacked once: y[i][e] = SiLU(bias[e] + sum_jj w[e][jj] x[i + jj][e]), the taps
// summed in order jj = 0..3 (w[c][3] hits the newest row).
template <typename TIn, int R>
__device__ __forceinline__ void conv_rows(bool conv, const u32x4_t (&xr)[R + 3], const u32x4_t (&wp)[4],
                                          const float (&bias)[Elem<TIn>::kVec], float (&y)[R][Elem<TIn>::kVec]) {
    constexpr int VEC = Elem<TIn>::kVec;
    if (conv) {
        float wv[4 * VEC], xs[R + 3][VEC];
#pragma unroll
        for (int m = 0; m < 4; m++) Elem<TIn>::unpack16(to_uint4(wp[m]), wv + m * VEC);
#pragma unroll
        for (int jj = 0; jj < R + 3; jj++) Elem<TIn>::unpack16(to_uint4(xr[jj]), xs[jj]);
#pragma unroll
        for (int i = 0; i < R; i++)
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                float acc = bias[e];
#pragma unroll
                for (int jj = 0; jj < 4; jj++) acc += wv[4 * e + jj] * xs[i + jj][e];
                y[i][e] = silu(acc);
            }
    } else {
#pragma unroll
        for (int i = 0; i < R; i++) Elem<TIn>::unpack16(to_uint4(xr[i + 3]), y[i]);
    }
}

// Raw 16-byte rows r0-3 .. r0+R-1 of one channel group for the chunk starting
// at token c0 (L valid rows; the sequence starts at bos).  Rows before the
// sequence start come from the conv state `hist` (3 inputs per channel,
// oldest first; channel e of the group at hist + 3 e) or are zero; rows at or
// past L are zero.  Without the conv only rows r0.. are read.
template <typename TIn, int R>
__device__ __forceinline__ void load_rows(u32x4_t (&x)[R + 3], const TIn* base, int64_t stride, int64_t c0,
                                          int r0, int L, int64_t bos, bool conv, const TIn* hist) {
#pragma unroll
    for (int j = 0; j < R + 3; j++) {
        const int row = r0 - 3 + j;
        const int64_t tt = c0 + row;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row < L && (conv || j >= 3)) {
            if (tt >= bos) {
                v = *reinterpret_cast<const u32x4_t*>(base + tt * stride);
            } else if (hist) {
                uint4 u = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < Elem<TIn>::kVec; e++) Elem<TIn>::set16(u, e, hist + 3 * e + (3 + (tt - bos)));
                v = to_u32x4(u);
            }
        }
        x[j] = v;
    }
}

// Pool entry holding sequence n's states: state_indices[n] (-1: none), or n
// itself without an index map.  Its stored states are the sequence's initial
// ones unless has_initial[n] is 0.
__device__ __forceinline__ int state_slot(const PrefillParams& p, int n) {
    return p.state_indices ? p.state_indices[n] : n;
}
__device__ __forceinline__ bool slot_has_initial(const PrefillParams& p, int n, int slot) {
    return slot >= 0 && (!p.has_initial || p.has_initial[n] != 0);
}

// Bias of one 16-byte channel group as raw element bits (0 without a bias):
// converted only where it is used, so that the load does not have to be
// waited for right away.
template <typename TIn>
__device__ __forceinline__ void conv_bias_raw(const PrefillParams& p, int64_t ch, uint32_t (&braw)[Elem<TIn>::kVec]) {
    const TIn* cb = static_cast<const TIn*>(p.conv_b);
#pragma unroll
    for (int e = 0; e < Elem<TIn>::kVec; e++) braw[e] = 0u;
    if (p.conv_width == 4 && cb) {
#pragma unroll
        for (int e = 0; e < Elem<TIn>::kVec; e++) {
            if constexpr (sizeof(TIn) == 2) braw[e] = uint32_t(cb[ch + e]) << 16;
            else braw[e] = __float_as_uint(cb[ch + e]);
        }
    }
}

// The 4 conv taps and the bias of one 16-byte channel group starting at
// channel ch, kept in registers by the workgroup.
template <typename TIn>
__device__ __forceinline__ void conv_params(const PrefillParams& p, int64_t ch, u32x4_t (&wp)[4],
                                            float (&bias)[Elem<TIn>::kVec]) {
    constexpr int VEC = Elem<TIn>::kVec;
    const TIn* cw = static_cast<const TIn*>(p.conv_w);
    const TIn* cb = static_cast<const TIn*>(p.conv_b);
#pragma unroll
    for (int m = 0; m < 4; m++) wp[m] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < VEC; e++) bias[e] = 0.0f;
    if (p.conv_width == 4) {
#pragma unroll
        for (int m = 0; m < 4; m++) wp[m] = *reinterpret_cast<const u32x4_t*>(cw + ch * 4 + m * VEC);
        if (cb) {
#pragma unroll
            for (int e = 0; e < VEC; e++) bias[e] = Elem<TIn>::get(cb + ch + e);
        }
    }
}

// ---------------------------------------------------------------- products

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

// Column block J of T = (I + A)^{-1} below the diagonal:
//   T_iJ = -T_ii sum_{k=J}^{i-1} A_ik T_kJ,  i = J+1 .. 3,
// from the diagonal inverses in Td; blocks (J..3, J) are written to Tf.
// Block products on fp32 matrix-core steps, in a fixed order.
template <int J, int PF, int PD>
__device__ __forceinline__ void inverse_column(const float* Af, const float* Td, float* Tf, int lr, int lg) {
    float4_t tc[4];
#pragma unroll
    for (int e = 0; e < 4; e++) tc[J][e] = Td[(16 * J + 4 * lg + e) * PD + lr];
#pragma unroll
    for (int i = J + 1; i < 4; i++) {
        float4_t s = kZero4;
#pragma unroll
        for (int k = J; k < i; k++) mma_blk_f32(s, Af + 16 * i * PF + 16 * k, PF, tc[k]);
        float4_t t = kZero4;
        mma_blk_f32(t, Td + 16 * i * PD, PD, s);
        tc[i] = -t;
    }
#pragma unroll
    for (int i = J; i < 4; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) Tf[(16 * i + 4 * lg + e) * PF + 16 * J + lr] = tc[i][e];
}

// e^x rounded to fp32 for an fp64 argument: x log2(e) is reduced in fp64 to an
// integer n and a fraction |f| <= 1/2, 2^f comes from the hardware exp2 and
// 2^n is applied exactly.  Relative error ~1.5e-7, against ~4e-6 for the fp32
// exponential of an fp32-rounded argument near -50.
__device__ __forceinline__ float exp_of_f64(double x) {
    const double t = x * 1.4426950408889634;
    const double n = rint(t);
    return ldexpf(__builtin_amdgcn_exp2f(static_cast<float>(t - n)), static_cast<int>(n));
}

// Split 8 consecutive fp32 values into 16-byte hi and lo packs.
template <typename E>
__device__ __forceinline__ void split_pack(const float (&x)[8], uint4& hi, uint4& lo) {
    const SFrag<E> f = split8<E>(x);
    hi = *reinterpret_cast<const uint4*>(&f.hi);
    lo = *reinterpret_cast<const uint4*>(&f.lo);
}

// ---------------------------------------------------------------- chunk map

// chunk_base[n] = sum_{m<n} ceil(len_m / 64), chunk_base[N] = total chunks.
// One workgroup scans the sequences in tiles of 256.
__global__ void __launch_bounds__(256) chunk_map_kernel(const int32_t* __restrict__ cu, int32_t n,
                                                         int32_t* __restrict__ base) {
    __shared__ int32_t s[256];
    const int t = threadIdx.x;
    int32_t carry = 0;
    for (int t0 = 0; t0 < n; t0 += 256) {
        const int i = t0 + t;
        const int32_t c = i < n ? int32_t((int64_t(cu[i + 1]) - cu[i] + kChunk - 1) / kChunk) : 0;
        s[t] = c;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int32_t x = t >= o ? s[t - o] : 0;
            __syncthreads();
            s[t] += x;
            __syncthreads();
        }
        if (i < n) base[i] = carry + s[t] - c;
        carry += s[255];
        __syncthreads();
    }
    if (t == 0) base[n] = carry;
}

// Descriptor of every chunk slot s < chunk_base[N]: {n, first token, length,
// first token of n}, n being the last sequence with chunk_base[n] <= s (the
// sequence that owns the slot; empty sequences own none).
__global__ void __launch_bounds__(256) slot_map_kernel(const int32_t* __restrict__ cu, int32_t n,
                                                        const int32_t* __restrict__ base,
                                                        int4* __restrict__ desc) {
    const int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (s >= base[n]) return;
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (base[mid] <= s) lo = mid;
        else hi = mid - 1;
    }
    const int32_t bos = cu[lo], c0 = bos + int32_t(s - base[lo]) * kChunk;
    const int32_t left = cu[lo + 1] - c0;
    desc[s] = int4{lo, c0, left < kChunk ? left : kChunk, bos};
}

// Sequences ordered by descending chunk count (ties by index), so that the
// longest dependent chains start first.  Ranks are unique, so the map is a
// permutation for any cu_seqlens contents.  The order only schedules work:
// results do not depend on it.  Beyond kMaxRanked sequences the quadratic
// ranking is skipped and the identity order used.
constexpr int kMaxRanked = 8192;
__global__ void __launch_bounds__(256) order_kernel(const int32_t* __restrict__ cu, int32_t n,
                                                     int32_t* __restrict__ order) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (n > kMaxRanked) {
        order[i] = i;
        return;
    }
    const int64_t ci = (int64_t(cu[i + 1]) - cu[i] + kChunk - 1) / kChunk;
    int rank = 0;
    for (int j = 0; j < n; j++) {
        const int64_t cj = (int64_t(cu[j + 1]) - cu[j] + kChunk - 1) / kChunk;
        rank += (cj > ci) || (cj == ci && j < i);
    }
    order[rank] = i;
}

// The three maps above in one workgroup, for problems small enough that one
// workgroup's loops are short (kSmallMapSeqs sequences, kSmallMapSlots chunk
// slots): saves two launches.  Same integer results as the three kernels.
constexpr int kSmallMapSeqs = 512;
constexpr int64_t kSmallMapSlots = 65536;
__global__ void __launch_bounds__(256) small_map_kernel(const int32_t* __restrict__ cu, int32_t n,
                                                         int32_t* __restrict__ base, int32_t* __restrict__ order,
                                                         int4* __restrict__ desc) {
    __shared__ int32_t s[256];
    __shared__ int32_t sb[kSmallMapSeqs + 1];
    const int t = threadIdx.x;
    // chunk_base: the same tile scan as chunk_map_kernel, kept in LDS too
    int32_t carry = 0;
    for (int t0 = 0; t0 < n; t0 += 256) {
        const int i = t0 + t;
        const int32_t c = i < n ? int32_t((int64_t(cu[i + 1]) - cu[i] + kChunk - 1) / kChunk) : 0;
        s[t] = c;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int32_t x = t >= o ? s[t - o] : 0;
            __syncthreads();
            s[t] += x;
            __syncthreads();
        }
        if (i < n) {
            base[i] = carry + s[t] - c;
            sb[i] = carry + s[t] - c;
        }
        carry += s[255];
        __syncthreads();
    }
    if (t == 0) {
        base[n] = carry;
        sb[n] = carry;
    }
    __syncthreads();
    // order: rank by descending chunk count, ties by index
    for (int i = t; i < n; i += 256) {
        const int32_t ci = sb[i + 1] - sb[i];
        int rank = 0;
        for (int j = 0; j < n; j++) {
            const int32_t cj = sb[j + 1] - sb[j];
            rank += (cj > ci) || (cj == ci && j < i);
        }
        order[rank] = i;
    }
    // slot descriptors
    for (int64_t sl = t; sl < carry; sl += 256) {
        int lo = 0, hi = n - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sb[mid] <= sl) lo = mid;
            else hi = mid - 1;
        }
        const int32_t bos = cu[lo], c0 = bos + int32_t(sl - sb[lo]) * kChunk;
        const int32_t left = cu[lo + 1] - c0;
        desc[sl] = int4{lo, c0, left < kChunk ? left : kChunk, bos};
    }
}

// ---------------------------------------------------------------- segment split: chain map

// Chains of the segment split.  Sequence n of nch chunks runs as
// S = max(1, ceil(nch / seg)) chains; chain s covers chunks [s Ls, min((s + 1) Ls, nch))
// with Ls = ceil(nch / S), so the split depends on the sequence's length
// alone.  chain_base[n] = chains before sequence n (chain_base[N] = all),
// desc[c] = {sequence, first chunk, chunks, segment index}.  One workgroup
// scans the sequences in tiles of 256.
__global__ void __launch_bounds__(256) chain_map_kernel(const int32_t* __restrict__ cu, int32_t n, int32_t seg,
                                                         int32_t* __restrict__ chain_base, int4* __restrict__ desc) {
    __shared__ int32_t s[256];
    const int t = threadIdx.x;
    int32_t carry = 0;
    for (int t0 = 0; t0 < n; t0 += 256) {
        const int i = t0 + t;
        int32_t nch = 0, S = 0;
        if (i < n) {
            nch = int32_t((int64_t(cu[i + 1]) - cu[i] + kChunk - 1) / kChunk);
            S = nch > seg ? (nch + seg - 1) / seg : 1;
        }
        s[t] = S;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int32_t x = t >= o ? s[t - o] : 0;
            __syncthreads();
            s[t] += x;
            __syncthreads();
        }
        if (i < n) {
            const int32_t base = carry + s[t] - S, Ls = (nch + S - 1) / S;
            chain_base[i] = base;
            for (int32_t k = 0; k < S; k++) {
                const int32_t j0 = k * Ls, len = nch - j0 < Ls ? nch - j0 : Ls;
                desc[base + k] = int4{i, j0, len, k};
            }
        }
        carry += s[255];
        __syncthreads();
    }
    if (t == 0) chain_base[n] = carry;
}

// Chains ordered by descending length (ties by index), the longest dependent
// chains first; beyond kMaxRanked chains the identity order.  Scheduling
// only: results do not depend on it.
__global__ void __launch_bounds__(256) chain_order_kernel(const int32_t* __restrict__ count,
                                                           const int4* __restrict__ desc,
                                                           int32_t* __restrict__ order) {
    const int nc = *count;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nc) return;
    if (nc > kMaxRanked) {
        order[i] = i;
        return;
    }
    const int li = desc[i].z;
    int rank = 0;
    for (int j = 0; j < nc; j++) {
        const int lj = desc[j].z;
        rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
}

// ---------------------------------------------------------------- prep: q|k prologue and chunk-local terms

// Workgroup = (chunk slot, key head): 4 waves; two workgroups fit a CU (LDS
// below 80 KB, registers below 256 per lane), so one unit's barrier waits
// overlap the other's work.
constexpr int kPrepThreads = 256;

template <int DK, int VEC>
struct PrepSmem {
    // K planes (16-bit units; hi, lo) [token][d_k]: 72-word rows for d_k = 128
    // keep the Gram fragment reads free of bank conflicts
    static constexpr int kPitchK = DK == 128 ? DK + 16 : DK + 8;
    // Q planes, read once per unit: d_k + 8, whose two planes take exactly the
    // bytes of A and T that replace them after the Gram tiles
    static constexpr int kPitchQ = DK + 8;
    static constexpr int kPitchF = kChunk + 4;  // fp32 [token][token]
    static constexpr int kPitchD = 20;          // diagonal inverse blocks: [4][16][kPitchD]
    static constexpr int kNG = 2 * (DK / VEC);  // q|k 16-byte groups per row
    static constexpr int kRedCols = kNG < 32 ? kNG : 32;  // partial sums kept per row
    static constexpr size_t szK = size_t(kChunk) * kPitchK * sizeof(uint16_t);
    static constexpr size_t szQ = size_t(kChunk) * kPitchQ * sizeof(uint16_t);
    static constexpr size_t szF = size_t(kChunk) * kPitchF * sizeof(float);
    static constexpr size_t oKhi = 0, oKlo = szK;
    static constexpr size_t oX = 2 * szK;                       // Q hi, Q lo; then A, T (fp32)
    static constexpr size_t szX = 2 * szQ > 2 * szF ? 2 * szQ : 2 * szF;
    static constexpr size_t oQhi = oX, oQlo = oX + szQ, oA = oX, oT = oX + szF;
    static constexpr size_t oR = oX + szX;                      // partial sums; then Td, gam, bet
    static constexpr size_t szTd = size_t(4) * 16 * kPitchD * sizeof(float);
    static constexpr size_t szR0 = size_t(kChunk) * kRedCols * sizeof(float);
    static constexpr size_t szR1 = szTd + kChunk * (sizeof(double) + sizeof(float));
    static constexpr size_t oTd = oR, oGam = oR + szTd, oBet = oGam + kChunk * sizeof(double);
    static constexpr size_t kBytes = oR + (szR0 > szR1 ? szR0 : szR1);
    static_assert(2 * kBytes <= size_t(kLdsLimit), "two workgroups per CU");
    static_assert(oX % 16 == 0 && oQlo % 16 == 0 && oT % 16 == 0 && oR % 16 == 0 && oGam % 16 == 0 &&
                      oBet % 16 == 0,
                  "16-byte aligned regions");
};

// A 16-byte piece of a chunk image.  Nontemporal: the images of one call far
// exceed the L2 caches, and the carry kernel reads them only after the whole
// chunk-parallel kernel has run (measured ~1.5% faster per call than plain
// stores, mostly in the carry kernel's reads).
template <typename E>
__device__ __forceinline__ void img_store(E* dst, uint4 v) {
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(&v), reinterpret_cast<u32x4_t*>(dst));
}

template <int DK, typename TIn>
__global__ void __launch_bounds__(kPrepThreads, 2) prep_kernel(const PrefillParams p) {
    constexpr int VEC = Elem<TIn>::kVec;
    constexpr int NGQ = DK / VEC;          // 16-byte groups per q (or k) head row
    constexpr int NG = 2 * NGQ;
    constexpr int RB = kPrepThreads / NG;  // row blocks per chunk
    constexpr int RPB = kChunk / RB;       // rows per thread
    constexpr int KS = DK / 32;
    static_assert(kPrepThreads % NG == 0 && kChunk % RB == 0 && NG <= 64, "q|k prologue tiling");
    using S = PrepSmem<DK, VEC>;
    using E = typename OpFor<TIn>::type;
    typedef typename OpVec<E>::v8 V8;
    constexpr int PK = S::kPitchK, PQ = S::kPitchQ, PF = S::kPitchF, PD = S::kPitchD, RC = S::kRedCols;
    constexpr int PAIR = NG / RC;  // partial sums combined by lane pairs first (1 or 2)

    __shared__ __attribute__((aligned(16))) char smem[S::kBytes];
    E* Khi = reinterpret_cast<E*>(smem + S::oKhi);
    E* Klo = reinterpret_cast<E*>(smem + S::oKlo);
    E* Qhi = reinterpret_cast<E*>(smem + S::oQhi);
    E* Qlo = reinterpret_cast<E*>(smem + S::oQlo);
    float* Af = reinterpret_cast<float*>(smem + S::oA);
    float* Tf = reinterpret_cast<float*>(smem + S::oT);
    float* red = reinterpret_cast<float*>(smem + S::oR);
    float* Td = reinterpret_cast<float*>(smem + S::oTd);
    double* gam = reinterpret_cast<double*>(smem + S::oGam);
    float* bet = reinterpret_cast<float*>(smem + S::oBet);

    const int64_t units = int64_t(p.chunk_base[p.num_seqs]) * p.h_k;
    const int64_t u = blockIdx.x;
    if (u >= units) return;
    const int64_t cs = u / p.h_k;
    const int hk = int(u % p.h_k);
    const int4 d = reinterpret_cast<const int4*>(p.slot_desc)[cs];  // sequence, first token, length, start
    const int n = d.x, L = d.z;
    const int64_t c0 = d.y, bos = d.w;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int G = p.h_v / p.h_k;
    const int64_t nq = int64_t(p.h_k) * DK, C = 2 * nq + int64_t(p.h_v) * p.d_v;
    const bool conv = p.conv_width == 4;

    // ---- prologue: one 16-byte channel group of q|k over RPB consecutive rows
    //      per thread (the conv history rows and taps loaded once) ----
    const int pg = tid % NG, prow0 = (tid / NG) * RPB;
    const int pwhich = pg / NGQ, poff = (pg % NGQ) * VEC;
    float y[RPB][VEC];
    {
        const int64_t pch = (pwhich ? nq : 0) + int64_t(hk) * DK + poff;
        u32x4_t pw[4];
        float pbias[VEC];
        conv_params<TIn>(p, pch, pw, pbias);
        const TIn* pbase = static_cast<const TIn*>(pwhich ? p.k : p.q) + int64_t(hk) * DK + poff;
        u32x4_t xr[RPB + 3];
        if (c0 - 3 >= bos && L == kChunk) {
            // interior chunk: every row, history included, is in the sequence
#pragma unroll
            for (int jj = 0; jj < RPB + 3; jj++)
                xr[jj] = *reinterpret_cast<const u32x4_t*>(pbase + (c0 + prow0 - 3 + jj) * nq);
        } else {
            const int sl = state_slot(p, n);
            const TIn* hist = (p.conv_state_in && slot_has_initial(p, n, sl))
                                  ? static_cast<const TIn*>(p.conv_state_in) + (int64_t(sl) * C + pch) * 3
                                  : nullptr;
            load_rows<TIn, RPB>(xr, pbase, nq, c0, prow0, L, bos, conv, hist);
        }
        conv_rows<TIn, RPB>(conv, xr, pw, pbias, y);
    }
    // partial sums of squares per (row, group), pairs of neighbouring groups
    // combined first when there are more than 32 groups (commuted pairs: both
    // lanes hold the same sum)
#pragma unroll
    for (int i = 0; i < RPB; i++) {
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; e++) {
            if (prow0 + i >= L) y[i][e] = 0.0f;
            ss += y[i][e] * y[i][e];
        }
        if constexpr (PAIR == 2) ss += __shfl_xor(ss, 1);
        if (pg % PAIR == 0) red[(prow0 + i) * RC + pg / PAIR] = ss;
    }
    // the first value head's decays, by wave 0 after its share of the prologue
    auto decays = [&](int gi) {
        const int h = hk * G + gi;
        const bool in = lane < L;
        const int64_t at = (c0 + (in ? lane : 0)) * p.h_v + h;
        const float gv = in ? p.g[at] : 0.0f;
        const float bv = in ? beta_of(p.beta[at], p.beta_logits != 0) : 0.0f;
        double x = gv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double t = __shfl_up(x, o);
            if (lane >= o) x += t;
        }
        const double gl = __shfl(x, 63);
        gam[lane] = x;
        bet[lane] = bv;
        const float ex = exp_of_f64(x);
        float* sc = p.scal_img + (cs * p.h_v + h) * Img<DK>::kScal;
        sc[lane] = bv;
        sc[kChunk + lane] = ex;
        sc[2 * kChunk + lane] = exp_of_f64(gl - x);
        const float exl = __shfl(ex, 63);
        sc[3 * kChunk + lane] = lane == 0 ? exl : 0.0f;
    };
    lds_barrier();
    // normalised rows as split pairs into the K and Q planes and the K|Q
    // image; each thread sums its row's partial sums itself, in a fixed order
    {
        E* img = static_cast<E*>(p.kq_img) + (cs * p.h_k + hk) * Img<DK>::kKQ + (pwhich ? 0 : 2 * kChunk * DK);
        E* dhi = pwhich ? Khi : Qhi;
        E* dlo = pwhich ? Klo : Qlo;
        const int dp = pwhich ? PK : PQ;
        float sc[RPB];
#pragma unroll
        for (int i = 0; i < RPB; i++) {
            const float* rr = red + (prow0 + i) * RC + pwhich * (RC / 2);
            static_assert((RC / 2) % 4 == 0, "partial sums in 16-byte loads");
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < RC / 2; q += 4) {
                const float4 r4 = *reinterpret_cast<const float4*>(rr + q);
                sum += r4.x;
                sum += r4.y;
                sum += r4.z;
                sum += r4.w;
            }
            sc[i] = p.qk_l2norm ? 1.0f / sqrtf(sum + p.l2_eps) : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < RPB; i++) {
            const int row = prow0 + i;
            if constexpr (VEC == 8) {
                // bf16 pairs: 8 columns per plane piece
                bf16x2_t h16[VEC / 2], l16[VEC / 2];
#pragma unroll
                for (int e = 0; e < VEC / 2; e++)
                    split2(y[i][2 * e] * sc[i], y[i][2 * e + 1] * sc[i], h16[e], l16[e]);
                const uint4 hv = *reinterpret_cast<const uint4*>(h16), lv = *reinterpret_cast<const uint4*>(l16);
                *reinterpret_cast<uint4*>(dhi + row * dp + poff) = hv;
                *reinterpret_cast<uint4*>(dlo + row * dp + poff) = lv;
                img_store(img + row * DK + poff, hv);
                img_store(img + kChunk * DK + row * DK + poff, lv);
            } else {
                // fp32 values: columns 8c .. 8c+3 go to the hi plane and
                // 8c+4 .. 8c+7 to the lo plane, at the piece of columns 8c
                const float4 v = make_float4(y[i][0] * sc[i], y[i][1] * sc[i], y[i][2] * sc[i], y[i][3] * sc[i]);
                const int c8 = poff & ~7;
                const bool second = (poff & 4) != 0;
                *reinterpret_cast<float4*>((second ? dlo : dhi) + row * dp + c8) = v;
                img_store(img + (second ? kChunk * DK : 0) + row * DK + c8, *reinterpret_cast<const uint4*>(&v));
            }
        }
    }
    lds_barrier();

    // ---- Gram tiles of this wave's tile row: K K^T and Q K^T, tiles (w, t),
    //      t <= w, raw fp32 in accumulator layout (the A operands read once) ----
    float4_t kk[4], qk[4];
    {
        SFrag<E> kf[KS], qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            kf[ks] = lds_sfrag(Khi, Klo, PK, 16 * w + lr, 32 * ks + 8 * lg);
            qf[ks] = lds_sfrag(Qhi, Qlo, PQ, 16 * w + lr, 32 * ks + 8 * lg);
        }
#pragma unroll
        for (int t = 0; t < 4; t++) kk[t] = qk[t] = kZero4;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if (t < w) {
                    const SFrag<E> b = lds_sfrag(Khi, Klo, PK, 16 * t + lr, 32 * ks + 8 * lg);
                    mma3(kk[t], kf[ks], b);
                    mma3(qk[t], qf[ks], b);
                } else if (t == w) {
                    mma3(kk[t], kf[ks], kf[ks]);
                    mma3(qk[t], qf[ks], kf[ks]);
                }
            }
    }
    if (w == 0) decays(0);  // gam, bet: the partial sums' bytes are free now
    lds_barrier();          // the Q planes are free for A and T; the first decays are in

    // ---- per value head of the group ----
    for (int gi = 0; gi < G; gi++) {
        const int h = hk * G + gi;
        const int64_t ih = cs * p.h_v + h;
        if (gi > 0) {
            if (w == 0) decays(gi);
            lds_barrier();
        }
        // A (fp32, LDS) and P (fp32, LDS) from the Gram tiles in registers:
        // A[r][s] = beta_r e^{gam_r - gam_s} (k_r . k_s) for s < r,
        // P[r][s] = e^{gam_r - gam_s} (q_r . k_s) for s <= r
        {
            double gr[4];
            float br[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                gr[e] = gam[16 * w + 4 * lg + e];
                br[e] = bet[16 * w + 4 * lg + e];
            }
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if (t > w) continue;
                const int sidx = 16 * t + lr;
                const double gs = gam[sidx];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 16 * w + 4 * lg + e;
                    const float ex = __expf(static_cast<float>(gr[e] - gs));
                    const float dec = sidx <= r ? ex : 0.0f;
                    Af[r * PF + sidx] = sidx < r ? br[e] * dec * kk[t][e] : 0.0f;
                    Tf[r * PF + sidx] = sidx <= r ? dec * qk[t][e] : 0.0f;
                }
            }
        }
        lds_barrier();
        // P image (lower blocks, 8 columns per item), then the inverses of the
        // 16x16 diagonal blocks of (I + A) by forward substitution (wave 0, one
        // column per lane)
        {
            E* pimg = static_cast<E*>(p.tp_img) + ih * Img<DK>::kTP + 2 * TriPack::kPieces * 8;
#pragma unroll
            for (int it = 0; it < 2; it++) {
                const int item = tid + 256 * it;
                const int r = item >> 3, s0 = (item & 7) * 8;
                if ((s0 >> 4) <= (r >> 4)) {
                    float pp[8];
                    *reinterpret_cast<float4*>(pp) = *reinterpret_cast<const float4*>(Tf + r * PF + s0);
                    *reinterpret_cast<float4*>(pp + 4) = *reinterpret_cast<const float4*>(Tf + r * PF + s0 + 4);
                    uint4 hv, lv;
                    split_pack<E>(pp, hv, lv);
                    const int q = TriPack::row_start(r) + (s0 >> 3);
                    img_store(pimg + 8 * q, hv);
                    img_store(pimg + 8 * (TriPack::kPieces + q), lv);
                }
            }
        }
        if (w == 0) {
            const int b = lane >> 4, c = lane & 15;
            // column-oriented: once x[r] is known it is added into every later
            // row's sum, so the steps of one column are independent (each row
            // still sums s = 0, 1, ..., r - 1 in order)
            float x[16], acc[16];
#pragma unroll
            for (int r = 0; r < 16; r++) acc[r] = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                x[r] = (r < c) ? 0.0f : ((r == c) ? 1.0f : -acc[r]);
#pragma unroll
                for (int s2 = r + 1; s2 < 16; s2++) acc[s2] += Af[(16 * b + s2) * PF + 16 * b + r] * x[r];
            }
#pragma unroll
            for (int r = 0; r < 16; r++) Td[(16 * b + r) * PD + c] = x[r];
        }
        lds_barrier();
        // off-diagonal blocks of T on fp32 matrix cores, one column block per wave
        if (w == 0) {
            inverse_column<0, PF, PD>(Af, Td, Tf, lr, lg);
        } else if (w == 1) {
            inverse_column<1, PF, PD>(Af, Td, Tf, lr, lg);
        } else if (w == 2) {
            inverse_column<2, PF, PD>(Af, Td, Tf, lr, lg);
        } else if (lane < 16) {  // block (3, 3) is its diagonal inverse
#pragma unroll
            for (int r = 0; r < 16; r++) Tf[(48 + r) * PF + 48 + lane] = Td[(48 + r) * PD + lane];
        }
        lds_barrier();
        // T image (lower blocks)
        {
            E* timg = static_cast<E*>(p.tp_img) + ih * Img<DK>::kTP;
#pragma unroll
            for (int it = 0; it < 2; it++) {
                const int item = tid + 256 * it;
                const int r = item >> 3, s0 = (item & 7) * 8;
                if ((s0 >> 4) <= (r >> 4)) {
                    float tl[8];
                    *reinterpret_cast<float4*>(tl) = *reinterpret_cast<const float4*>(Tf + r * PF + s0);
                    *reinterpret_cast<float4*>(tl + 4) = *reinterpret_cast<const float4*>(Tf + r * PF + s0 + 4);
                    float t8[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) t8[e] = ((s0 + e) >> 4 <= (r >> 4)) ? tl[e] : 0.0f;
                    uint4 hv, lv;
                    split_pack<E>(t8, hv, lv);
                    const int q = TriPack::row_start(r) + (s0 >> 3);
                    img_store(timg + 8 * q, hv);
                    img_store(timg + 8 * (TriPack::kPieces + q), lv);
                }
            }
        }
        // the next value head's decays touch only gam, bet and the scalar
        // image, whose last readers came before the previous barrier; its A and
        // P writes come after the barrier that follows the decays
    }
}

// ---------------------------------------------------------------- carry: v prologue, state chain, outputs

// Raw buffer resources: word 3 of the descriptor for untyped 32-bit accesses
// on gfx9-family parts.  A raw access at or past num_records bytes is out of
// range: a store is dropped, a load returns zero.
constexpr int kBufferFlags = 0x00020000;

template <typename T> __device__ __forceinline__ void buf_put(__amdgpu_buffer_rsrc_t r, int off, float x);
template <> __device__ __forceinline__ void buf_put<float>(__amdgpu_buffer_rsrc_t r, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}

// ---------------------------------------------------------------- carry: the state chain

// Workgroup = (sequence, value head, 64-column slice of d_v), 8 waves in two
// roles, so that the work off the state's dependent path runs beside it:
// waves 0-3 ("main") hold the state columns [16w, 16w + 16) in matrix-core
// accumulators for the whole sequence and compute K H, R, D = T R and the
// update;
// wave 4 + w ("helper") covers the same columns and does the rest of the
// staging (T|P images, scalars, conv + SiLU of v) and its loads, Q H, P D and
// the output.  The K|Q image goes through the main waves' registers (a helper
// holding it too would exceed its 256 registers).  Per chunk, three
// workgroup barriers:
//   stage:  all waves write the chunk to LDS; main also splits the state
//           operand and hands it to the helpers through LDS; the helpers
//           convolve half of the chunk's v rows.
//   B:      main: K H, R, D = T R; D's split operand goes to LDS (over this
//           wave's own columns of V, which only it reads).  helpers: Q H,
//           then conv + SiLU of the other half of the next chunk's v rows.
//   C:      main: the state update.  helpers: P D and the output rows.
// The helpers issue their part of the next chunk's loads as phase B starts;
// the main waves request the next K|Q image in two halves during phase B
// (after K H, and after D's operand is written).
// The two roles run separate loops with the same barriers, so their register
// live ranges do not overlap.
constexpr int kCarryThreads = 512;

template <int DK>
struct CarrySmem {
    // K, Q image rows (16-bit).  Fragment reads (16 rows, one 16-byte piece
    // each) measured bank-conflict-free on gfx950 with 72-word rows (d_k = 128)
    // and at half speed with the 68-word rows of d_k + 8.
    static constexpr int kPitchK = DK == 128 ? DK + 16 : DK + 8;
    // T, P image rows (16-bit): 64 columns unpadded, 16-byte pieces swizzled
    // by row (tp_off), which measured conflict-free where 72-column rows did not
    static constexpr int kPitchT = kChunk;
    static constexpr int kPitchV = kDvs + 4;    // V rows (fp32); D's operand afterwards
    static constexpr int KS = DK / 32;
    static constexpr size_t szKQ = size_t(kChunk) * kPitchK * sizeof(uint16_t);
    static constexpr size_t szTP = size_t(kChunk) * kPitchT * sizeof(uint16_t);
    static constexpr size_t oKQ = 0;         // K hi, K lo, Q hi, Q lo
    static constexpr size_t oTP = 4 * szKQ;  // T hi, T lo, P hi, P lo
    static constexpr size_t oV = oTP + 4 * szTP;
    static constexpr size_t oScal = oV + size_t(kChunk) * kPitchV * sizeof(float);
    static constexpr size_t oHB = oScal + Img<DK>::kScal * sizeof(float);  // [wave][ks][hi|lo][lane] 16 B
    static constexpr size_t kBytes = oHB + size_t(4) * KS * 2 * 64 * 16;
    static_assert(kBytes <= size_t(kLdsLimit), "LDS budget");
    static_assert(oTP % 16 == 0 && oV % 16 == 0 && oScal % 16 == 0 && oHB % 16 == 0, "16-byte aligned regions");
    static_assert(kPitchV * 4 % 16 == 0 && 4 * 16 * (kPitchV * 4) >= 4 * 64 * 16, "D operand fits V's rows");
};

// Element offset of (row, col) in a T|P plane of the carry kernel: 64-column
// rows whose 16-byte pieces are XOR-swizzled by row % 8.
__device__ __forceinline__ int tp_off(int row, int col) {
    return row * kChunk + ((((col >> 3) ^ row) & 7) << 3) + (col & 7);
}
template <typename E>
__device__ __forceinline__ SFrag<E> tp_frag(const E* hi, const E* lo, int row, int k) {
    typedef typename OpVec<E>::v8 V8;
    const int o = tp_off(row, k);
    SFrag<E> f;
    f.hi = *reinterpret_cast<const V8*>(hi + o);
    f.lo = *reinterpret_cast<const V8*>(lo + o);
    return f;
}

// Products whose B operand comes from accumulators, in the carry's chain.
// Within a 32-deep k-step a product may take its k indices in any order that
// A and B share.  For bf16 operands T R, P D and the state update take, for
// lane group g = l / 16, k = k0 + 4 g + i (i < 4) and k0 + 16 + 4 g + i - 4
// (i >= 4): the rows an accumulator pair (rows k0 .. k0 + 15, k0 + 16 .. k0 +
// 31) already holds in lane l, so the B operand needs no lane exchange, and
// the A operand is read in two 8-byte halves (the update's transposed reads
// are 8-byte reads either way): 265 -> 253 us for the carry at 4 x 4096
// tokens.  K H and Q H keep the K-major order (acc_to_operand on the state):
// with their 16 A fragments per k-step read in halves the carry took 411 us.
// fp32 operands keep the K-major order throughout.
template <typename E>
__device__ __forceinline__ SFrag<E> acc_pair_operand(const float4_t& t0, const float4_t& t1) {
    float x[8];
    if constexpr (__is_same(E, F32Op)) {
        acc_to_operand(t0, t1, x);
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            x[e] = t0[e];
            x[e + 4] = t1[e];
        }
    }
    return split8<E>(x);
}
template <typename E>
__device__ __forceinline__ SFrag<E> tp_frag_acc(const E* hi, const E* lo, int row, int k0, int g) {
    if constexpr (__is_same(E, F32Op)) {
        return tp_frag(hi, lo, row, k0 + 8 * g);
    } else {
        const int o0 = tp_off(row, k0 + 4 * g), o1 = tp_off(row, k0 + 16 + 4 * g);
        SFrag<E> f;
        f.hi = __builtin_shufflevector(*reinterpret_cast<const bf16x4_t*>(hi + o0),
                                       *reinterpret_cast<const bf16x4_t*>(hi + o1), 0, 1, 2, 3, 4, 5, 6, 7);
        f.lo = __builtin_shufflevector(*reinterpret_cast<const bf16x4_t*>(lo + o0),
                                       *reinterpret_cast<const bf16x4_t*>(lo + o1), 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
}
// K^T operand (transposed LDS read) in that k order
template <typename E>
__device__ __forceinline__ SFrag<E> lds_sfrag_tr_acc(const E* hi, const E* lo, int pitch, int k0, int g, int col0) {
    if constexpr (__is_same(E, F32Op)) {
        return lds_sfrag_tr(hi, lo, pitch, k0 + 8 * g, col0);
    } else {
        const int j = threadIdx.x & 15;
        const int off = (k0 + 4 * g + (j >> 2)) * pitch + col0 + 4 * (j & 3);
        SFrag<E> f;
        f.hi = __builtin_shufflevector(lds_tr16(hi + off), lds_tr16(hi + off + 16 * pitch), 0, 1, 2, 3, 4, 5, 6, 7);
        f.lo = __builtin_shufflevector(lds_tr16(lo + off), lds_tr16(lo + off + 16 * pitch), 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
}

// Byte offset, in the V region, of piece p (0..3: D k-step 0 hi, lo, k-step 1
// hi, lo) of lane l of column block w: row 16 p + l % 16, 16 bytes at 16 (l/16)
// within bytes [64 w, 64 w + 64) of the row, which hold exactly V's columns
// [16 w, 16 w + 16).  Lanes 0-15 of one access take 16 rows (measured fewer
// bank conflicts in the kernel than 4 lanes per row; 16 rows of 68 words
// still run at half the conflict-free rate, but V's row pitch serves its own
// reads without conflicts).
template <int PV>
__device__ __forceinline__ int dop_offset(int w, int piece, int l) {
    return (16 * piece + (l & 15)) * (PV * 4) + 64 * w + 16 * (l >> 4);
}

template <int DK, int DV, typename TIn, typename TOut, bool CH>
__global__ void __launch_bounds__(kCarryThreads, 1) carry_kernel(const PrefillParams p) {
    constexpr int NS = DV / kDvs, NSK = DK / kDvs;
    constexpr int HT = kCarryThreads / 2;                 // helper threads
    constexpr int VEC = Elem<TIn>::kVec;
    constexpr int NGV = kDvs / VEC;                    // 16-byte groups of a v slice row
    constexpr int VRPB = kChunk / (HT / NGV);          // v rows per helper thread
    constexpr int KT = DK / 16, KS = DK / 32;
    constexpr int NKQ = Img<DK>::kKQ / 8 / HT;         // 16-byte K|Q pieces per main thread
    constexpr int NTP = Img<DK>::kTP / 8 / HT;         // 16-byte T|P pieces per helper thread
    static_assert(Img<DK>::kKQ % (8 * HT) == 0 && Img<DK>::kTP % (8 * HT) == 0, "image pieces");
    static_assert(NTP * HT == 4 * TriPack::kPieces, "T|P pieces");
    static_assert(Img<DK>::kScal == HT, "one scalar per helper thread");
    static_assert(HT % NGV == 0 && kChunk % (HT / NGV) == 0, "v prologue tiling");
    static_assert(DV % kDvs == 0, "d_v slices");
    using S = CarrySmem<DK>;
    using E = typename OpFor<TIn>::type;
    typedef typename OpVec<E>::v8 V8;
    constexpr int PK = S::kPitchK, PT = S::kPitchT, PV = S::kPitchV;

    __shared__ __attribute__((aligned(16))) char smem[S::kBytes];
    E* kq = reinterpret_cast<E*>(smem + S::oKQ);
    E* tp = reinterpret_cast<E*>(smem + S::oTP);
    const E* Khi = kq;
    const E* Klo = kq + kChunk * PK;
    const E* Qhi = kq + 2 * kChunk * PK;
    const E* Qlo = kq + 3 * kChunk * PK;
    const E* Thi = tp;
    const E* Tlo = tp + kChunk * PT;
    const E* Phi = tp + 2 * kChunk * PT;
    const E* Plo = tp + 3 * kChunk * PT;
    float* Vf = reinterpret_cast<float*>(smem + S::oV);
    char* dop = smem + S::oV;
    float* scal = reinterpret_cast<float*>(smem + S::oScal);
    char* hbs = smem + S::oHB;
    const float* bet = scal;
    const float* eg = scal + kChunk;
    const float* dl = scal + 2 * kChunk;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cw = wave & 3;  // column block of this wave (main and helper alike)
    const int lr = lane & 15, lg = lane >> 4;
    // XCD-aware unit map: workgroup b runs on XCD b % 8; the M members of
    // group g = (order index, key head) share XCD g % 8.  Without the segment
    // split a group is a (sequence, key head) with M = G NS members, the value
    // heads' d_v slices.  With it (CH) a group is a (chain, key head) and has
    // G NSK more members: the identity chains of the d_k columns.
    const int G = p.h_v / p.h_k, M = G * (CH ? NS + NSK : NS);
    const int ngroups = (CH ? p.chain_base[p.num_seqs] : p.num_seqs) * p.h_k;
    const int xcd = int(blockIdx.x & 7u), kx = int(blockIdx.x >> 3);
    const int grp = (kx / M) * 8 + xcd, mem = kx % M;
    if (grp >= ngroups) return;
    const bool ident = CH && mem >= G * NS;  // an identity chain (segment split only)
    const int mrel = ident ? mem - G * NS : mem, nsl = ident ? NSK : NS;
    const int hk = grp % p.h_k, gi = mrel / nsl, slice = mrel % nsl;
    // The chain: sequence n's chunks [j0, j0 + nch), segment segi of nseg.
    int n, j0 = 0, nch = 0, chain = 0, segi = 0, nseg = 1;
    if constexpr (CH) {
        chain = p.chain_order[grp / p.h_k];
        const int4 d = reinterpret_cast<const int4*>(p.chain_desc)[chain];
        n = d.x;
        j0 = d.y;
        nch = d.z;
        segi = d.w;
        nseg = p.chain_base[n + 1] - p.chain_base[n];
        if (ident && segi == 0) return;  // the first segment starts from the true state
    } else {
        n = p.order[grp / p.h_k];
    }
    const int h = hk * G + gi;
    const int wcol = 16 * cw + lr;        // this lane's column within the slice
    const int col = slice * kDvs + wcol;  // ... and within d_v (d_k for an identity chain)
    const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
    if constexpr (!CH) nch = int((eos - bos + kChunk - 1) / kChunk);
    const int cb = p.chunk_base[n] + j0;               // chunk slot of the chain's first chunk
    const int64_t tok0 = bos + int64_t(j0) * kChunk;  // its first token
    const int slot = state_slot(p, n);
    const bool has_init = slot_has_initial(p, n, slot);
    // A value chain of a split sequence leaves its final state in seg_state
    // (the combine kernel chains them); segments after the first start from
    // zero and write their outputs to seg_oloc (the correction kernel adds
    // their dependence on the start state); an identity chain runs from the
    // d_k identity columns with zero v, leaving the segment's transition in
    // seg_trans and its outputs in seg_y.
    const bool split = CH && nseg > 1;

    if (wave < 4) {
        // ======== main waves: the state and its dependent chain ========
        const int64_t state_base = (int64_t(slot) * p.h_v + h) * DK * DV + col;  // used only when slot >= 0
        // State column: hacc[it][e] = H[16 it + 4 lg + e][col].
        float4_t hacc[KT];
#pragma unroll
        for (int it = 0; it < KT; it++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int row = 16 * it + 4 * lg + e;
                if (ident)
                    hacc[it][e] = row == col ? 1.0f : 0.0f;
                else
                    hacc[it][e] = (p.initial_state && has_init && segi == 0)
                                      ? p.initial_state[state_base + int64_t(row) * DV] : 0.0f;
            }
        u32x4_t pkq[NKQ];
        auto fetch_kq = [&](int j, int i0, int i1) {
            const u32x4_t* skq = reinterpret_cast<const u32x4_t*>(static_cast<const E*>(p.kq_img) +
                                                                  ((int64_t(cb) + j) * p.h_k + hk) * Img<DK>::kKQ);
#pragma unroll
            for (int i = 0; i < NKQ; i++)
                if (i >= i0 && i < i1) pkq[i] = skq[tid + HT * i];
        };
        if (nch > 0) fetch_kq(0, 0, NKQ);

        for (int j = 0; j < nch; j++) {
            // ---- stage: the K|Q image, and the state as the B operand (also handed to the helpers) ----
#pragma unroll
            for (int i = 0; i < NKQ; i++) {
                const int pc = tid + HT * i;  // piece: plane, row, 8 columns
                const int plane = pc / (kChunk * DK / 8), rem = pc % (kChunk * DK / 8);
                *reinterpret_cast<u32x4_t*>(kq + plane * kChunk * PK + (rem / (DK / 8)) * PK + 8 * (rem % (DK / 8))) =
                    pkq[i];
            }
            SFrag<E> hb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                float x[8];
                acc_to_operand(hacc[2 * ks], hacc[2 * ks + 1], x);
                hb[ks] = split8<E>(x);
                *reinterpret_cast<V8*>(hbs + (((cw * KS + ks) * 2 + 0) * 64 + lane) * 16) = hb[ks].hi;
                *reinterpret_cast<V8*>(hbs + (((cw * KS + ks) * 2 + 1) * 64 + lane) * 16) = hb[ks].lo;
            }
            lds_barrier();

            // ---- B: R = beta (V - e^gam K H), D = T R; D's operand to LDS ----
            float4_t rr[4];
#pragma unroll
            for (int tb = 0; tb < 4; tb++) {
                float4_t kh = kZero4;
#pragma unroll
                for (int ks = 0; ks < KS; ks++) mma3(kh, lds_sfrag(Khi, Klo, PK, 16 * tb + lr, 32 * ks + 8 * lg), hb[ks]);
                const float4 egv = *reinterpret_cast<const float4*>(eg + 16 * tb + 4 * lg);
                const float4 btv = *reinterpret_cast<const float4*>(bet + 16 * tb + 4 * lg);
                const float egr[4] = {egv.x, egv.y, egv.z, egv.w}, btr[4] = {btv.x, btv.y, btv.z, btv.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 16 * tb + 4 * lg + e;
                    rr[tb][e] = btr[e] * (Vf[r * PV + wcol] - egr[e] * kh[e]);
                }
            }
            // The next chunk's K|Q image, half of it here, once K H has read this
            // chunk's planes, half after D's operand is written.  Issued right
            // after the staging barrier, with the helpers' T|P, scalar and v
            // loads, the two queued in the CU's vector memory pipeline and
            // delayed the helpers' Q H; all of it here, or half or all in phase C,
            // measured slower (the issue on the chain, or the data late for the
            // next staging).
            if (j + 1 < nch) fetch_kq(j + 1, 0, NKQ / 2);
            float4_t dd[4];
            {
                SFrag<E> rb[2];
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    rb[s] = acc_pair_operand<E>(rr[2 * s], rr[2 * s + 1]);
                }
#pragma unroll
                for (int tb = 0; tb < 4; tb++) {
                    dd[tb] = kZero4;
#pragma unroll
                    for (int ks = 0; ks <= tb / 2; ks++) mma3(dd[tb], tp_frag_acc(Thi, Tlo, 16 * tb + lr, 32 * ks, lg), rb[ks]);
                }
            }
            // D's operand overwrites this wave's own V columns, which only this
            // wave has read (R above, on which D depends).
#pragma unroll
            for (int s = 0; s < 2; s++) {
                const SFrag<E> f = acc_pair_operand<E>(dd[2 * s], dd[2 * s + 1]);
                *reinterpret_cast<V8*>(dop + dop_offset<PV>(cw, 2 * s, lane)) = f.hi;
                *reinterpret_cast<V8*>(dop + dop_offset<PV>(cw, 2 * s + 1, lane)) = f.lo;
            }
            if (j + 1 < nch) fetch_kq(j + 1, NKQ / 2, NKQ);
            lds_barrier();

            // ---- C: H <- e^{gam_last} H + K^T diag(e^{gam_last - gam}) D ----
            {
                SFrag<E> ab[2];
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    float4_t a0, a1;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int r0 = 32 * s + 4 * lg + e, r1 = r0 + 16;
                        a0[e] = dl[r0] * dd[2 * s][e];
                        a1[e] = dl[r1] * dd[2 * s + 1][e];
                    }
                    ab[s] = acc_pair_operand<E>(a0, a1);
                }
                const float decay = scal[3 * kChunk];
#pragma unroll
                for (int it = 0; it < KT; it++) {
                    hacc[it] *= decay;
#pragma unroll
                    for (int s = 0; s < 2; s++) mma3(hacc[it], lds_sfrag_tr_acc(Khi, Klo, PK, 32 * s, lg, 16 * it), ab[s]);
                }
            }
            lds_barrier();
        }

        if (split || ident) {
            const int rs = ident ? DK : DV;  // row stride of the segment buffers
            float* dst = (ident ? p.seg_trans : p.seg_state) + (int64_t(chain) * p.h_v + h) * DK * rs + col;
#pragma unroll
            for (int it = 0; it < KT; it++)
#pragma unroll
                for (int e = 0; e < 4; e++) dst[int64_t(16 * it + 4 * lg + e) * rs] = hacc[it][e];
        } else if (p.final_state && slot >= 0) {
#pragma unroll
            for (int it = 0; it < KT; it++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    p.final_state[state_base + int64_t(16 * it + 4 * lg + e) * DV] = hacc[it][e];
        }
    } else {
        // ======== helper waves: staging, loads, Q H, P D and the output ========
        const int ht = tid - HT;
        const int64_t nq = int64_t(p.h_k) * DK, nv = int64_t(p.h_v) * DV, C = 2 * nq + nv;
        const bool conv = p.conv_width == 4;
        TOut* out = static_cast<TOut*>(p.o);
        // v prologue: one 16-byte channel group of the slice for VRPB rows
        const int vg = ht % NGV, vrow0 = (ht / NGV) * VRPB;
        const int64_t vch = 2 * nq + int64_t(h) * DV + slice * kDvs + vg * VEC;
        const TIn* vbase = static_cast<const TIn*>(p.v) + int64_t(h) * DV + slice * kDvs + vg * VEC;
        const TIn* vhist = (p.conv_state_in && has_init)
                               ? static_cast<const TIn*>(p.conv_state_in) + (int64_t(slot) * C + vch) * 3 : nullptr;
        u32x4_t vwp[4];
        float vbias[VEC];
        if (ident) {  // no v channels: an identity slice may lie past d_v
#pragma unroll
            for (int m = 0; m < 4; m++) vwp[m] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < VEC; e++) vbias[e] = 0.0f;
        } else {
            conv_params<TIn>(p, vch, vwp, vbias);
        }

        u32x4_t ptp[NTP], xv[VRPB + 3];
        float psc;
        // The next chunk's T|P pieces, scalars and raw v rows (issued once the
        // chunk is staged, consumed at the next staging).
        auto fetch = [&](int j) {
            const int64_t cslot = int64_t(cb) + j;
            const u32x4_t* stp = reinterpret_cast<const u32x4_t*>(static_cast<const E*>(p.tp_img) +
                                                                  (cslot * p.h_v + h) * Img<DK>::kTP);
            psc = p.scal_img[(cslot * p.h_v + h) * Img<DK>::kScal + ht];
            const int64_t c0 = tok0 + int64_t(j) * kChunk;
            if (ident) {
                // no v: the identity columns start with zero inputs
            } else if (c0 - 3 >= bos && c0 + kChunk <= eos) {
                // interior chunk: every row, history included, is in the sequence
#pragma unroll
                for (int jj = 0; jj < VRPB + 3; jj++)
                    xv[jj] = *reinterpret_cast<const u32x4_t*>(vbase + (c0 + vrow0 - 3 + jj) * nv);
            } else {
                const int L = int(eos - c0 < kChunk ? eos - c0 : kChunk);
                load_rows<TIn, VRPB>(xv, vbase, nv, c0, vrow0, L, bos, conv, vhist);
            }
#pragma unroll
            for (int i = 0; i < NTP; i++) ptp[i] = stp[ht + HT * i];
        };
        // Blocks (0, 1) and (2, 3) of the T and P planes are read by the
        // products (k-steps of 32 columns) but never staged: zero them once.
        for (int i = ht; i < 4 * 2 * 16 * 2; i += HT) {
            const int plane = i >> 6, blk = (i >> 5) & 1, rr = (i >> 1) & 15, half = i & 1;
            const int r = 32 * blk + rr, c = 32 * blk + 16 + 8 * half;
            *reinterpret_cast<u32x4_t*>(tp + plane * kChunk * PT + tp_off(r, c)) = u32x4_t{0u, 0u, 0u, 0u};
        }
        // LDS offsets of this thread's T|P pieces (the same every chunk)
        int tpo[NTP];
#pragma unroll
        for (int i = 0; i < NTP; i++) {
            const int pc = ht + HT * i;
            int r, c8;
            TriPack::locate(pc % TriPack::kPieces, r, c8);
            tpo[i] = (pc / TriPack::kPieces) * kChunk * PT + tp_off(r, 8 * c8);
        }
        // conv(4) + SiLU of this thread's v rows of chunk j (zero past its end),
        // computed from the raw rows during the previous chunk's phase C
        // Half of the rows (h = 1) are convolved during the previous chunk's
        // phase C, the other half (h = 0) while staging, which balances both
        // roles at both barriers.
        constexpr int VH = VRPB / 2;
        static_assert(VRPB % 2 == 0, "v rows in two halves");
        float vy[VRPB][VEC];
        auto conv_v = [&](int j, int h) {
            const int64_t c0 = tok0 + int64_t(j) * kChunk;
            const int L = int(eos - c0 < kChunk ? eos - c0 : kChunk);
            float y[VH][VEC];
            conv_rows<TIn, VH>(conv, *reinterpret_cast<const u32x4_t(*)[VH + 3]>(xv + h * VH), vwp, vbias, y);
#pragma unroll
            for (int i = 0; i < VH; i++)
#pragma unroll
                for (int e = 0; e < VEC; e++)
                    vy[h * VH + i][e] = (vrow0 + h * VH + i < L && !ident) ? y[i][e] : 0.0f;
        };
        if (nch > 0) {
            fetch(0);
            conv_v(0, 1);
        }

        // fp32 outputs of the segment split: identity chains to seg_y (d_k
        // columns), value chains after the first segment to seg_oloc
        float* fo = nullptr;
        int fcols = DV;
        if constexpr (CH) {
            if (ident) {
                fo = p.seg_y;
                fcols = DK;
            } else if (segi > 0) {
                fo = p.seg_oloc;
            }
        }

        for (int j = 0; j < nch; j++) {
            const int64_t c0 = tok0 + int64_t(j) * kChunk;
            const int L = int(eos - c0 < kChunk ? eos - c0 : kChunk);

            // ---- stage the chunk (every wave is done with the previous one) ----
#pragma unroll
            for (int i = 0; i < NTP; i++) *reinterpret_cast<u32x4_t*>(tp + tpo[i]) = ptp[i];
            scal[ht] = psc;
            conv_v(j, 0);
            // 16-byte stores (scalar ones collided 8-way on the banks)
#pragma unroll
            for (int i = 0; i < VRPB; i++)
#pragma unroll
                for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<float4*>(Vf + (vrow0 + i) * PV + vg * VEC + e) =
                        make_float4(vy[i][e], vy[i][e + 1], vy[i][e + 2], vy[i][e + 3]);
            lds_barrier();
            if (j + 1 < nch) fetch(j + 1);

            // ---- B: e^gam Q H from the state operand the main wave left in LDS ----
            float4_t eqh[4];
            {
                SFrag<E> hb[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    hb[ks].hi = *reinterpret_cast<const V8*>(hbs + (((cw * KS + ks) * 2 + 0) * 64 + lane) * 16);
                    hb[ks].lo = *reinterpret_cast<const V8*>(hbs + (((cw * KS + ks) * 2 + 1) * 64 + lane) * 16);
                }
#pragma unroll
                for (int tb = 0; tb < 4; tb++) {
                    float4_t qh = kZero4;
#pragma unroll
                    for (int ks = 0; ks < KS; ks++) mma3(qh, lds_sfrag(Qhi, Qlo, PK, 16 * tb + lr, 32 * ks + 8 * lg), hb[ks]);
                    const float4 egv = *reinterpret_cast<const float4*>(eg + 16 * tb + 4 * lg);
                    const float egr[4] = {egv.x, egv.y, egv.z, egv.w};
#pragma unroll
                    for (int e = 0; e < 4; e++) eqh[tb][e] = egr[e] * qh[e];
                }
            }
            // half of the next chunk's v conv (its raw rows were requested at
            // the start of this phase), in the time the main waves' phase B
            // takes beyond Q H
            if (j + 1 < nch) conv_v(j + 1, 1);
            lds_barrier();

            // ---- C: o = scale (e^gam Q H + P D) ----
            {
                // The chunk's rows of o through a buffer resource whose extent ends
                // after row L - 1: the hardware drops the stores of rows past the
                // sequence's end, so no store needs a branch of its own.
                const __amdgpu_buffer_rsrc_t orsrc =
                    (CH && fo) ? __builtin_amdgcn_make_buffer_rsrc(fo + c0 * p.h_v * fcols, short(0),
                                                                   L * p.h_v * fcols * int(sizeof(float)), kBufferFlags)
                               : __builtin_amdgcn_make_buffer_rsrc(out + c0 * p.h_v * DV, short(0),
                                                                   L * p.h_v * DV * int(sizeof(TOut)), kBufferFlags);
                SFrag<E> db[2];
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    db[s].hi = *reinterpret_cast<const V8*>(dop + dop_offset<PV>(cw, 2 * s, lane));
                    db[s].lo = *reinterpret_cast<const V8*>(dop + dop_offset<PV>(cw, 2 * s + 1, lane));
                }
#pragma unroll
                for (int tb = 0; tb < 4; tb++) {
                    float4_t pd = kZero4;
#pragma unroll
                    for (int ks = 0; ks <= tb / 2; ks++) mma3(pd, tp_frag_acc(Phi, Plo, 16 * tb + lr, 32 * ks, lg), db[ks]);
                    float val[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) val[e] = p.scale * (eqh[tb][e] + pd[e]);
                    if (CH && fo) {
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int r = 16 * tb + 4 * lg + e;
                            buf_put<float>(orsrc, ((r * p.h_v + h) * fcols + col) * int(sizeof(float)), val[e]);
                        }
                    } else if constexpr (sizeof(TOut) == 2) {
                        // Lanes lr and lr ^ 1 hold columns 2c and 2c + 1 of the same
                        // rows: the even lane takes rows 4 lg + 0, 1 and the odd lane
                        // rows 4 lg + 2, 3 of both columns, converted two at a time
                        // (round to nearest even) and stored as 4-byte pairs.
                        const bool odd = (lr & 1) != 0;
                        const float q0 = __shfl_xor(odd ? val[0] : val[2], 1);
                        const float q1 = __shfl_xor(odd ? val[1] : val[3], 1);
                        const float2_t a = odd ? float2_t{q0, val[2]} : float2_t{val[0], q0};
                        const float2_t b = odd ? float2_t{q1, val[3]} : float2_t{val[1], q1};
                        const int r = 16 * tb + 4 * lg + (odd ? 2 : 0), c2 = col & ~1;
                        const bf16x2_t pa = __builtin_convertvector(a, bf16x2_t);
                        const bf16x2_t pb = __builtin_convertvector(b, bf16x2_t);
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pa), orsrc,
                                                              ((r * p.h_v + h) * DV + c2) * 2, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pb), orsrc,
                                                              (((r + 1) * p.h_v + h) * DV + c2) * 2, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int r = 16 * tb + 4 * lg + e;
                            buf_put<TOut>(orsrc, ((r * p.h_v + h) * DV + col) * int(sizeof(TOut)), val[e]);
                        }
                    }
                }
            }
            lds_barrier();
        }

        // Final conv state: the sequence's last 3 raw inputs for this
        // workgroup's v channels and, in its group's first member, the key
        // head's q and k channels; a sequence shorter than 3 reaches into its
        // conv history.  Both are entry `slot` of their arrays (nothing is
        // written without one).  Every history read of these channels came
        // before (q and k: the chunk-local kernel; v: this workgroup's first
        // chunk), and one thread reads a channel's three values before writing
        // them, so the output may be the history buffer itself.  With the
        // segment split the first segment's chain writes it: it is the one
        // that reads the v history, and a later segment running beside it
        // could otherwise overwrite that history before it is read.
        if (p.conv_state_out && conv && slot >= 0 && !ident && segi == 0) {
            const int64_t len = eos - bos;
            const TIn* csi = (p.conv_state_in && has_init) ? static_cast<const TIn*>(p.conv_state_in) : nullptr;
            TIn* cso = static_cast<TIn*>(p.conv_state_out);
            const int nch_out = kDvs + (mem == 0 ? 2 * DK : 0);
            for (int i = ht; i < nch_out; i += HT) {
                int64_t c, stride;
                const TIn* src;
                if (i < kDvs) {
                    c = 2 * nq + int64_t(h) * DV + slice * kDvs + i;
                    src = static_cast<const TIn*>(p.v) + (c - 2 * nq);
                    stride = nv;
                } else if (i < kDvs + DK) {
                    c = int64_t(hk) * DK + (i - kDvs);
                    src = static_cast<const TIn*>(p.q) + c;
                    stride = nq;
                } else {
                    c = nq + int64_t(hk) * DK + (i - kDvs - DK);
                    src = static_cast<const TIn*>(p.k) + (c - nq);
                    stride = nq;
                }
                const int64_t at = (int64_t(slot) * C + c) * 3;
                TIn vals[3];
#pragma unroll
                for (int jj = 0; jj < 3; jj++) {
                    const int64_t pos = len - 3 + jj;
                    vals[jj] = pos >= 0 ? src[(bos + pos) * stride] : (csi ? csi[at + 3 + pos] : TIn(0));
                }
#pragma unroll
                for (int jj = 0; jj < 3; jj++) cso[at + jj] = vals[jj];
            }
        }
    }
}

// ---------------------------------------------------------------- segment split: combine and correct

// Step 2 of the segment split, per (split sequence, value head, 16 columns
// of d_v): the segments' start states in order.  H_1 = the first segment's
// final state; H_{s+1} = M_s H_s + F_s, with M_s the segment's transition
// (seg_trans) and F_s its final state from a zero start (seg_state).  H_s
// replaces F_s in seg_state (the correction reads it) and the last H is the
// sequence's final state.  fp32; each element's products are summed over d_k
// in order, all of a thread's rows at once (independent accumulators).  16
// columns per workgroup (64 measured 22.6 us at one 32768-token sequence:
// too few workgroups for the chip).
constexpr int kCombineCols = 16;
template <int DK, int DV>
__global__ void __launch_bounds__(256) segment_combine_kernel(const PrefillParams p) {
    constexpr int CC = kCombineCols, NS = DV / CC, RGN = 256 / CC, RPT = DK / RGN;
    __shared__ __attribute__((aligned(16))) float Ms[DK][DK + 4];
    __shared__ float Hs[DK][CC];
    const int b = int(blockIdx.x);
    const int slice = b % NS, h = (b / NS) % p.h_v, n = b / (NS * p.h_v);
    const int c0 = p.chain_base[n], nseg = p.chain_base[n + 1] - c0;
    if (nseg <= 1) return;
    const int t = threadIdx.x, cc = t % CC, rg = t / CC;  // column; rows rg + RGN r
    float H[RPT];
    const int64_t colofs = int64_t(slice) * CC + cc;
    const float* f0 = p.seg_state + (int64_t(c0) * p.h_v + h) * DK * DV + colofs;
#pragma unroll
    for (int r = 0; r < RPT; r++) H[r] = f0[int64_t(rg + RGN * r) * DV];
    for (int sg = 1; sg < nseg; sg++) {
        const int64_t c = c0 + sg;
        __syncthreads();  // the previous segment's reads of Ms and Hs are done
#pragma unroll
        for (int r = 0; r < RPT; r++) Hs[rg + RGN * r][cc] = H[r];
        const float4* m = reinterpret_cast<const float4*>(p.seg_trans + (c * p.h_v + h) * DK * DK);
        for (int i = t; i < DK * DK / 4; i += 256)
            *reinterpret_cast<float4*>(&Ms[i / (DK / 4)][4 * (i % (DK / 4))]) = m[i];
        float* fs = p.seg_state + (c * p.h_v + h) * DK * DV + colofs;
        float acc[RPT];
#pragma unroll
        for (int r = 0; r < RPT; r++) acc[r] = 0.0f;
        __syncthreads();
        for (int k = 0; k < DK; k += 4) {
            const float h0 = Hs[k][cc], h1 = Hs[k + 1][cc], h2 = Hs[k + 2][cc], h3 = Hs[k + 3][cc];
#pragma unroll
            for (int r = 0; r < RPT; r++) {
                const float4 mv = *reinterpret_cast<const float4*>(&Ms[rg + RGN * r][k]);
                acc[r] = fmaf(mv.x, h0, acc[r]);
                acc[r] = fmaf(mv.y, h1, acc[r]);
                acc[r] = fmaf(mv.z, h2, acc[r]);
                acc[r] = fmaf(mv.w, h3, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            const float f = fs[int64_t(rg + RGN * r) * DV];
            fs[int64_t(rg + RGN * r) * DV] = H[r];  // start state of segment sg
            H[r] = acc[r] + f;
        }
    }
    const int slot = state_slot(p, n);
    if (p.final_state && slot >= 0) {
        float* fin = p.final_state + (int64_t(slot) * p.h_v + h) * DK * DV + colofs;
#pragma unroll
        for (int r = 0; r < RPT; r++) fin[int64_t(rg + RGN * r) * DV] = H[r];
    }
}

// Step 3 of the segment split, per (8 consecutive chunk slots, value head):
// for each chunk of a segment s >= 1, o = O_loc + Y H_s, where O_loc
// (seg_oloc) is the segment's output from a zero start, Y (seg_y) the output
// of its identity columns (o's dependence on the start state) and H_s its
// start state.  Y H_s runs on the matrix cores with the operands of the
// chain's own products (split bf16 or fp32): wave w takes rows 16 w .. 16 w
// + 15 of the chunk across all of d_v, so Y is read once; H_s waits in LDS
// as ready operand fragments, staged again only when the segment changes.
// Each chunk's loads are issued during the previous chunk's products, before
// its stores: the vector memory counter retires loads and stores in order, so
// a load issued behind stores could only be used once they completed.
constexpr int kCorrectChunks = 8;
template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(256) segment_correct_kernel(const PrefillParams p) {
    constexpr int KS = DK / 32, NTT = DV / 16;  // k-steps; 16-column tiles of d_v
    using E = typename OpFor<TIn>::type;
    typedef typename OpVec<E>::v8 V8;
    // H_s fragments: [ks][tile][hi, lo][lane], 16 bytes each
    __shared__ __attribute__((aligned(16))) char hbs[KS * NTT * 2 * 64 * 16];
    const int h = int(blockIdx.x % unsigned(p.h_v));
    const int64_t g0 = int64_t(blockIdx.x / unsigned(p.h_v)) * kCorrectChunks;
    const int64_t nslots = p.chunk_base[p.num_seqs];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 15, lg = lane >> 4;
    const int64_t ystride = int64_t(p.h_v) * DK, ostride = int64_t(p.h_v) * DV;
    // The next chunk of this group that needs the correction (its first
    // token, chain and rows; c0 < 0 when none is left), found by scalar loads
    // ahead of time, so that its rows can be requested while the previous
    // chunk's products run.
    struct Item { int64_t c0, chain; int L; };
    auto next_item = [&](int& i) {
        for (; i < kCorrectChunks; i++) {
            const int64_t cs = g0 + i;
            if (cs >= nslots) break;
            const int4 d = reinterpret_cast<const int4*>(p.slot_desc)[cs];  // sequence, first token, length, start
            const int cbn = p.chain_base[d.x], nseg = p.chain_base[d.x + 1] - cbn;
            if (nseg <= 1) continue;
            const int ls = reinterpret_cast<const int4*>(p.chain_desc)[cbn].z;  // chunks per segment (the first is full)
            const int sg = int((int64_t(d.y) - d.w) / kChunk) / ls;
            if (sg == 0) continue;
            i++;
            return Item{int64_t(d.y), int64_t(cbn) + sg, d.z};
        }
        i = kCorrectChunks;
        return Item{-1, -1, 0};
    };
    // loads of one chunk: this wave's 16 rows of Y (row 16 w + lr, 8
    // consecutive k per k-step) and of O_loc (rows 16 w + 4 lg + e, column
    // 16 tile + lr)
    const int arow = 16 * w + lr;
    auto load = [&](const Item& it, float4 (&yv)[KS][2], float (&res)[NTT][4]) {
        const float* __restrict__ y = p.seg_y + (it.c0 * p.h_v + h) * DK;
        const float* __restrict__ ol = p.seg_oloc + (it.c0 * p.h_v + h) * DV;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++)
                yv[ks][hh] = arow < it.L ? *reinterpret_cast<const float4*>(y + arow * ystride + 32 * ks + 8 * lg + 4 * hh)
                                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int tile = 0; tile < NTT; tile++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 16 * w + 4 * lg + e;
                res[tile][e] = r < it.L ? ol[r * ostride + 16 * tile + lr] : 0.0f;
            }
    };
    float4 yv[KS][2], yn[KS][2];
    float res[NTT][4], rn[NTT][4];
    int pos = 0;
    Item nx = next_item(pos);
    if (nx.c0 >= 0) load(nx, yn, rn);
    int64_t cur = -1;  // the chain whose start state hbs holds
    while (nx.c0 >= 0) {
        const Item it = nx;
        nx = next_item(pos);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) yv[ks][0] = yn[ks][0], yv[ks][1] = yn[ks][1];
#pragma unroll
        for (int tile = 0; tile < NTT; tile++)
#pragma unroll
            for (int e = 0; e < 4; e++) res[tile][e] = rn[tile][e];
        if (it.chain != cur) {  // uniform over the workgroup
            __syncthreads();
            const float* src = p.seg_state + (it.chain * p.h_v + h) * DK * DV;
            for (int f = t; f < KS * NTT * 64; f += 256) {
                const int ks = f / (NTT * 64), tile = (f / 64) % NTT, l = f % 64;
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; e++) x[e] = src[(32 * ks + 8 * (l >> 4) + e) * DV + 16 * tile + (l & 15)];
                const SFrag<E> fr = split8<E>(x);
                *reinterpret_cast<V8*>(hbs + (((ks * NTT + tile) * 2 + 0) * 64 + l) * 16) = fr.hi;
                *reinterpret_cast<V8*>(hbs + (((ks * NTT + tile) * 2 + 1) * 64 + l) * 16) = fr.lo;
            }
            __syncthreads();
            cur = it.chain;
        }
        // the next chunk's rows, requested before this chunk's stores
        if (nx.c0 >= 0) load(nx, yn, rn);
        SFrag<E> a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const float x[8] = {yv[ks][0].x, yv[ks][0].y, yv[ks][0].z, yv[ks][0].w,
                                yv[ks][1].x, yv[ks][1].y, yv[ks][1].z, yv[ks][1].w};
            a[ks] = split8<E>(x);
        }
#pragma unroll
        for (int tile = 0; tile < NTT; tile++) {
            float4_t acc = kZero4;
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                SFrag<E> hb;
                hb.hi = *reinterpret_cast<const V8*>(hbs + (((ks * NTT + tile) * 2 + 0) * 64 + lane) * 16);
                hb.lo = *reinterpret_cast<const V8*>(hbs + (((ks * NTT + tile) * 2 + 1) * 64 + lane) * 16);
                mma3(acc, a[ks], hb);
            }
#pragma unroll
            for (int e = 0; e < 4; e++) res[tile][e] += acc[e];
        }
        TOut* __restrict__ out = static_cast<TOut*>(p.o) + (it.c0 * p.h_v + h) * DV;
#pragma unroll
        for (int tile = 0; tile < NTT; tile++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 16 * w + 4 * lg + e;
                if (r < it.L) Elem<TOut>::put(out + r * ostride + 16 * tile + lr, res[tile][e]);
            }
    }
}

hipError_t record(void* const* events, int i, hipStream_t stream) {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) : hipSuccess;
}

template <int DK, int DV, typename TIn, typename TOut, bool CH>
hipError_t run(const PrefillParams& p, hipStream_t stream, void* const* events) {
    hipError_t err = record(events, 0, stream);
    if (err != hipSuccess) return err;
    if (p.slots > 0) {
        // one workgroup per (chunk slot, key head); slots past the last chunk exit
        prep_kernel<DK, TIn><<<dim3(unsigned(p.slots * p.h_k)), dim3(kPrepThreads), 0, stream>>>(p);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    err = record(events, 1, stream);
    if (err != hipSuccess) return err;
    carry_kernel<DK, DV, TIn, TOut, CH><<<dim3(unsigned(carry_blocks(p.max_chains, p.h_k, p.h_v, DK, DV, CH))),
                                         dim3(kCarryThreads), 0, stream>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = record(events, 2, stream);
    if (err != hipSuccess) return err;
    if constexpr (CH) {
        segment_combine_kernel<DK, DV>
            <<<dim3(unsigned(int64_t(p.num_seqs) * p.h_v * (DV / kCombineCols))), dim3(256), 0, stream>>>(p);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (p.slots > 0) {
            const int64_t groups = (p.slots + kCorrectChunks - 1) / kCorrectChunks;
            segment_correct_kernel<DK, DV, TIn, TOut><<<dim3(unsigned(groups * p.h_v)), dim3(256), 0, stream>>>(p);
            err = hipGetLastError();
        }
    }
    return err;
}

template <typename TIn, typename TOut>
hipError_t run_dtype(const PrefillParams& p, int d_k, int d_v, hipStream_t stream, void* const* events) {
    const bool ch = p.segment_chunks > 0;
    if (d_k == 128 && d_v == 128)
        return ch ? run<128, 128, TIn, TOut, true>(p, stream, events) : run<128, 128, TIn, TOut, false>(p, stream, events);
    if (d_k == 128 && d_v == 64)
        return ch ? run<128, 64, TIn, TOut, true>(p, stream, events) : run<128, 64, TIn, TOut, false>(p, stream, events);
    if (d_k == 64 && d_v == 128)
        return ch ? run<64, 128, TIn, TOut, true>(p, stream, events) : run<64, 128, TIn, TOut, false>(p, stream, events);
    if (d_k == 64 && d_v == 64)
        return ch ? run<64, 64, TIn, TOut, true>(p, stream, events) : run<64, 64, TIn, TOut, false>(p, stream, events);
    return hipErrorInvalidValue;
}

}  // namespace

// Workspace of gdn_prefill_varlen_noalloc: a static device array, one copy on
// every GPU the library runs on.  In host code its name stands for a host-side
// symbol, not a device address: the address of the current device's copy is
// looked up once per device with hipGetSymbolAddress, and only that address is
// passed to the kernels.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        err = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillParams& p, int d_k, int d_v, int qkv_dtype, int out_dtype,
                          hipStream_t stream, void* const* events) {
    if (p.num_seqs <= 0) {
        for (int i = 0; i < 4 && events; i++) {
            const hipError_t err = record(events, i, stream);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    }
    hipError_t err;
    if (p.num_seqs <= kSmallMapSeqs && p.slots <= kSmallMapSlots) {
        small_map_kernel<<<dim3(1), dim3(256), 0, stream>>>(p.cu_seqlens, p.num_seqs, p.chunk_base, p.order,
                                                            reinterpret_cast<int4*>(p.slot_desc));
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    } else {
        chunk_map_kernel<<<dim3(1), dim3(256), 0, stream>>>(p.cu_seqlens, p.num_seqs, p.chunk_base);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        order_kernel<<<dim3((p.num_seqs + 255) / 256), dim3(256), 0, stream>>>(p.cu_seqlens, p.num_seqs, p.order);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (p.slots > 0) {
            slot_map_kernel<<<dim3(unsigned((p.slots + 255) / 256)), dim3(256), 0, stream>>>(
                p.cu_seqlens, p.num_seqs, p.chunk_base, reinterpret_cast<int4*>(p.slot_desc));
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    }
    if (p.segment_chunks > 0) {
        chain_map_kernel<<<dim3(1), dim3(256), 0, stream>>>(p.cu_seqlens, p.num_seqs, p.segment_chunks, p.chain_base,
                                                            reinterpret_cast<int4*>(p.chain_desc));
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        chain_order_kernel<<<dim3(unsigned((p.max_chains + 255) / 256)), dim3(256), 0, stream>>>(
            p.chain_base + p.num_seqs, reinterpret_cast<const int4*>(p.chain_desc), p.chain_order);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (qkv_dtype == 1)
        err = out_dtype == 1 ? run_dtype<bf16_t, bf16_t>(p, d_k, d_v, stream, events)
                             : run_dtype<bf16_t, float>(p, d_k, d_v, stream, events);
    else
        err = out_dtype == 1 ? run_dtype<float, bf16_t>(p, d_k, d_v, stream, events)
                             : run_dtype<float, float>(p, d_k, d_v, stream, events);
    if (err != hipSuccess) return err;
    return record(events, 3, stream);
}

}  // namespace gdn
