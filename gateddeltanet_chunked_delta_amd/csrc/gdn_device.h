// Device-side helpers for the gfx950 GDN kernels: element conversion,
// 16-byte vector loads and the matrix-core operand fragments and steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float float4_t __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector (kept in registers across loop iterations,
// where a struct-typed uint4 array can end up in scratch memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 to_uint4(const u32x4_t& v) { return uint4{v[0], v[1], v[2], v[3]}; }
__device__ __forceinline__ u32x4_t to_u32x4(const uint4& v) { return u32x4_t{v.x, v.y, v.z, v.w}; }

// bf16 is carried as its uint16_t bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16-byte load
    __device__ __forceinline__ static float get(const float* p) { return *p; }
    __device__ __forceinline__ static void load16(const float* p, float* out) {
        float4 x = *reinterpret_cast<const float4*>(p);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    }
    __device__ __forceinline__ static void put(float* p, float x) { *p = x; }
    __device__ __forceinline__ static void unpack16(const uint4& u, float* out) {
        out[0] = __uint_as_float(u.x); out[1] = __uint_as_float(u.y);
        out[2] = __uint_as_float(u.z); out[3] = __uint_as_float(u.w);
    }
    // element e of a 16-byte pack
    __device__ __forceinline__ static void set16(uint4& u, int e, const float* p) {
        const uint32_t b = __float_as_uint(*p);
        if (e == 0) u.x = b; else if (e == 1) u.y = b; else if (e == 2) u.z = b; else u.w = b;
    }
};
template <> struct Elem<bf16_t> {
    static constexpr int kVec = 8;
    __device__ __forceinline__ static float get(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void load16(const bf16_t* p, float* out) {
        uint4 x = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void put(bf16_t* p, float x) { *p = f32_to_bf16(x); }
    __device__ __forceinline__ static void unpack16(const uint4& u, float* out) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void set16(uint4& u, int e, const bf16_t* p) {
        const uint32_t b = *p;
        uint32_t* w = (e < 4) ? ((e < 2) ? &u.x : &u.y) : ((e < 6) ? &u.z : &u.w);
        *w = (e & 1) ? ((*w & 0x0000ffffu) | (b << 16)) : ((*w & 0xffff0000u) | b);
    }
};

// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// accesses, not for its outstanding global loads and stores, so loads of later
// data and stores of finished outputs stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Matrix-core lane layout (16x16 output tile, K-step 32): lane l supplies
// A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16], e = 0..7, and owns
// D[4*(l/16) + i][l%16], i = 0..3.

// Write strength from a beta input: the value itself, or sigmoid(b) for raw
// gates (expf is the accurate library exponential; large |b| saturates to 0 or 1).
__device__ __forceinline__ float beta_of(float b, bool logits) { return logits ? 1.0f / (1.0f + expf(-b)) : b; }

// y * sigmoid(y) with the hardware exp2 and reciprocal (a few ulp); large
// negative y gives exp = inf and a zero reciprocal, so the result is -0.
__device__ __forceinline__ float silu(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// ---- matrix-core operands ----
// Every product A B runs on the matrix cores from "fragments": lane l holds 8
// consecutive K-index values of one row of A (or one column of B), k = 8 (l/16)
// + e, e = 0..7, in two 16-byte halves `hi` and `lo`.  Two kinds:
//  * split bf16 (bf16-input calls): x ~= hi + lo with hi = bf16(x) and
//    lo = bf16(x - hi), both rounded to nearest even; a product takes three
//    16x16x32 bf16 steps, lo*hi + hi*lo + hi*hi (lo*lo is dropped), fp32
//    accumulation.  The pair keeps about 16 significant bits
//    (|x - hi - lo| <= 2^-16 |x|) over the whole fp32 range.
//  * fp32 (fp32-input calls): the 8 values themselves, `hi` = elements 0..3
//    and `lo` = elements 4..7; a product takes eight 16x16x4 fp32 steps, step e
//    multiplying element e of each lane's A and B values (its four k indices,
//    e, 8 + e, 16 + e, 24 + e, one per 16-lane group), fp32 accumulation.
//    Full fp32 range and precision, at a sixteenth of the bf16 rate.
// Both kinds take 32 bytes per lane and fragment, so LDS and workspace images
// have one layout: planes of 16-bit units, 16-byte pieces of 8 columns, the
// hi plane holding the first and the lo plane the second 16 bytes of each.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// 16-bit storage unit of fp32 operand planes (an fp32 value takes two).
struct alignas(2) F32Op {
    uint16_t bits;
};

template <typename E> struct OpVec;
template <> struct OpVec<__bf16> { typedef bf16x8_t v8; };
template <> struct OpVec<F32Op> { typedef float4_t v8; };

// Operand kind for each input element type.
template <typename TIn> struct OpFor;
template <> struct OpFor<float> { typedef F32Op type; };
template <> struct OpFor<bf16_t> { typedef __bf16 type; };

template <typename E>
struct SFrag {
    typename OpVec<E>::v8 hi, lo;
};

// bf16 split of the value pair (x0, x1); element 0 of each result belongs to
// x0.  The residual x - hi is exact in fp32 (hi keeps the leading 8 bits of x).
__device__ __forceinline__ void split2(float x0, float x1, bf16x2_t& hi, bf16x2_t& lo) {
    const float2_t v = {x0, x1};
    hi = __builtin_convertvector(v, bf16x2_t);
    const float2_t b = __builtin_convertvector(hi, float2_t);
    lo = __builtin_convertvector(float2_t{x0 - b[0], x1 - b[1]}, bf16x2_t);
}

template <typename E>
__device__ __forceinline__ SFrag<E> split8(const float (&x)[8]) {
    SFrag<E> f;
    if constexpr (__is_same(E, F32Op)) {
        f.hi = float4_t{x[0], x[1], x[2], x[3]};
        f.lo = float4_t{x[4], x[5], x[6], x[7]};
    } else {
        bf16x2_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; i++) split2(x[2 * i], x[2 * i + 1], h[i], l[i]);
        f.hi = bf16x8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
        f.lo = bf16x8_t{l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
    }
    return f;
}

// acc += A B over one 32-deep K step.
__device__ __forceinline__ void mma3(float4_t& acc, const SFrag<__bf16>& a, const SFrag<__bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma3(float4_t& acc, const SFrag<F32Op>& a, const SFrag<F32Op>& b) {
#pragma unroll
    for (int e = 0; e < 4; e++) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; e++) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], acc, 0, 0, 0);
}

constexpr float4_t kZero4 = {0.0f, 0.0f, 0.0f, 0.0f};

// Fragment from row-major hi/lo LDS matrices (8 consecutive elements along K).
template <typename E>
__device__ __forceinline__ SFrag<E> lds_sfrag(const E* hi, const E* lo, int pitch, int row, int k) {
    typedef typename OpVec<E>::v8 V8;
    SFrag<E> f;
    f.hi = *reinterpret_cast<const V8*>(hi + row * pitch + k);
    f.lo = *reinterpret_cast<const V8*>(lo + row * pitch + k);
    return f;
}

// Fragment whose K index runs down the rows of row-major hi/lo LDS matrices:
// element e is M[k + e][col0 + l%16].  bf16 planes are read with the gfx950
// LDS transpose load (ds_read_b64_tr_b16), 4 instructions.  Within each
// 16-lane group the load treats the 8-byte chunks addressed by lanes 0..15 as
// a 16x4 matrix M and returns M[j/4 + 4m][j%4], m = 0..3, to lane j.  So lane
// j addresses 4 consecutive columns col0 + 4 (j%4) .. of row k + j/4 and
// receives column col0 + j of rows k .. k+3; a second load covers rows
// k+4 .. k+7.  col0 is a multiple of 16 and the rows must be 8-byte aligned.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
// The loaded vectors are reinterpreted whole and joined with a shuffle: with
// ROCm 7.2's clang, extracting their 16-bit elements one by one produced code
// that kept only the first two elements of each load (checked on the GPU).
__device__ __forceinline__ bf16x4_t lds_tr16(const __bf16* p) {
    return __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p)));
}
__device__ __forceinline__ SFrag<__bf16> lds_sfrag_tr(const __bf16* hi, const __bf16* lo, int pitch, int k,
                                                      int col0) {
    const int j = threadIdx.x & 15;
    const int off = (k + (j >> 2)) * pitch + col0 + 4 * (j & 3);
    SFrag<__bf16> f;
    f.hi = __builtin_shufflevector(lds_tr16(hi + off), lds_tr16(hi + off + 4 * pitch), 0, 1, 2, 3, 4, 5, 6, 7);
    f.lo = __builtin_shufflevector(lds_tr16(lo + off), lds_tr16(lo + off + 4 * pitch), 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
}
// fp32 planes: column c of a row sits in plane (c & 4 ? lo : hi) at 16-bit
// offset (c & ~7) + 2 (c & 3); eight scalar reads.
__device__ __forceinline__ SFrag<F32Op> lds_sfrag_tr(const F32Op* hi, const F32Op* lo, int pitch, int k, int col0) {
    const int c = col0 + (threadIdx.x & 15);
    const F32Op* base = ((c & 4) ? lo : hi) + (c & ~7) + 2 * (c & 3);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = *reinterpret_cast<const float*>(base + (k + e) * pitch);
    return split8<F32Op>(x);
}

// Operand fragment from two accumulator tiles that hold rows [32s, 32s+16) and
// [32s+16, 32s+32) of a matrix X (lane l owns X[4*(l/16) + i][l%16] of each):
// returns x[e] = X[32s + 8*(l/16) + e][l%16], the K-major operand layout.
// permlane32_swap exchanges the upper half-wave of its first operand with the
// lower half-wave of its second; permlane16_swap exchanges the odd 16-lane rows
// of the first with the even rows of the second.
__device__ __forceinline__ void acc_to_operand(const float4_t& t0, const float4_t& t1, float (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(t0[e]), __float_as_uint(t1[e]), false, false);
        const auto t = __builtin_amdgcn_permlane16_swap(s[0], s[1], false, false);
        x[e] = __uint_as_float(t[0]);
        x[e + 4] = __uint_as_float(t[1]);
    }
}

}  // namespace gdn
