// Device-side helpers for the gfx950 GDN kernels: element conversion,
// 16-byte vector loads and the 16x16x32 matrix-core step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
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

// ---- split operands: x ~= hi + lo, both halves 16-bit matrix-core inputs ----
// A product of two split operands takes three 16-bit matrix-core steps,
// lo*hi + hi*lo + hi*hi (lo*lo is dropped), accumulated in fp32.  Two element
// types are used:
//  * bf16 (operands of bf16-input calls): hi = bf16(x), lo = bf16(x - hi),
//    both rounded to nearest even.  The pair keeps about 16 significant bits
//    (|x - hi - lo| <= 2^-16 |x|) over the whole fp32 range, and costs three
//    vector instructions per value (two values per packed conversion).
//  * fp16 (operands of fp32-input calls): hi = fp16(x), lo = fp16((x - hi) 2^11).
//    Scaling the residual by 2^11 keeps lo out of fp16's subnormal range, so
//    the pair keeps about 22 significant bits for 2^-14 <= |x| < 65504; the
//    cross terms go into a second accumulator that is scaled by 2^-11 at the end.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

template <typename E> struct OpVec;
template <> struct OpVec<_Float16> { typedef half8_t v8; typedef half4_t v4; };
template <> struct OpVec<__bf16> { typedef bf16x8_t v8; typedef bf16x4_t v4; };

// Operand element type for each input element type.
template <typename TIn> struct OpFor;
template <> struct OpFor<float> { typedef _Float16 type; };
template <> struct OpFor<bf16_t> { typedef __bf16 type; };

template <typename E>
struct SFrag {
    typename OpVec<E>::v8 hi, lo;
};

constexpr float kLoScale = 2048.0f;
constexpr float kLoUnscale = 1.0f / 2048.0f;

// fp16: hi is x converted by the hardware converter; the residual x - hi is
// then exact in fp32 (hi is converted back, so the pair always refers to the
// stored hi whatever rounding the converter applied) and is scaled by 2^11
// before its own conversion.  Values below fp16's normal range (2^-14) go
// entirely into lo: the matrix cores treat fp16 subnormal inputs as zero.
__device__ __forceinline__ _Float16 split_hi(float x) {
    return fabsf(x) < 6.103515625e-05f ? static_cast<_Float16>(0.0f) : static_cast<_Float16>(x);
}

// Splits of the value pair (x0, x1); element 0 of each result belongs to x0.
__device__ __forceinline__ void split2(float x0, float x1, half2_t& hi, half2_t& lo) {
    hi = half2_t{split_hi(x0), split_hi(x1)};
    lo = half2_t{static_cast<_Float16>((x0 - static_cast<float>(hi[0])) * kLoScale),
                 static_cast<_Float16>((x1 - static_cast<float>(hi[1])) * kLoScale)};
}
// bf16: the residual x - hi is exact in fp32 (hi keeps the leading 8 bits of x).
__device__ __forceinline__ void split2(float x0, float x1, bf16x2_t& hi, bf16x2_t& lo) {
    const float2_t v = {x0, x1};
    hi = __builtin_convertvector(v, bf16x2_t);
    const float2_t b = __builtin_convertvector(hi, float2_t);
    lo = __builtin_convertvector(float2_t{x0 - b[0], x1 - b[1]}, bf16x2_t);
}

template <typename E>
__device__ __forceinline__ SFrag<E> split8(const float (&x)[8]) {
    typedef typename OpVec<E>::v8 V8;
    typedef E V2 __attribute__((ext_vector_type(2)));
    V2 h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; i++) split2(x[2 * i], x[2 * i + 1], h[i], l[i]);
    SFrag<E> f;
    f.hi = V8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    f.lo = V8{l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
    return f;
}

// hh += A.hi B.hi; xx += A.lo B.hi + A.hi B.lo (the fp16 cross terms carry the
// 2^11 scale; the bf16 ones do not and go straight into hh).
__device__ __forceinline__ void mma3(float4_t& hh, float4_t& xx, const SFrag<_Float16>& a, const SFrag<_Float16>& b) {
    xx = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b.hi, xx, 0, 0, 0);
    xx = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.lo, xx, 0, 0, 0);
    hh = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.hi, hh, 0, 0, 0);
}
__device__ __forceinline__ void mma3(float4_t& hh, float4_t&, const SFrag<__bf16>& a, const SFrag<__bf16>& b) {
    hh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, hh, 0, 0, 0);
    hh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, hh, 0, 0, 0);
    hh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, hh, 0, 0, 0);
}

// The finished product.
template <typename E>
__device__ __forceinline__ float4_t combine(const float4_t& hh, const float4_t& xx) {
    if constexpr (__is_same(E, __bf16)) {
        return hh;
    } else {
        float4_t r;
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = hh[i] + xx[i] * kLoUnscale;
        return r;
    }
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
// element e is M[k + e][col0 + l%16], read with the gfx950 LDS transpose load
// (ds_read_b64_tr_b16), 4 instructions.  Within each 16-lane group the load treats
// the 8-byte chunks addressed by lanes 0..15 as a 16x4 matrix M and returns
// M[j/4 + 4m][j%4], m = 0..3, to lane j.  So lane j addresses 4 consecutive
// columns col0 + 4 (j%4) .. of row k + j/4 and receives column col0 + j of
// rows k .. k+3; a second load covers rows k+4 .. k+7.  col0 is a multiple of
// 16 and the rows must be 8-byte aligned.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
// The loaded vectors are reinterpreted whole and joined with a shuffle: with
// ROCm 7.2's clang, extracting their 16-bit elements one by one produced code
// that kept only the first two elements of each load (checked on the GPU).
template <typename E>
__device__ __forceinline__ typename OpVec<E>::v4 lds_tr16(const E* p) {
    return __builtin_bit_cast(typename OpVec<E>::v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p)));
}
template <typename E>
__device__ __forceinline__ SFrag<E> lds_sfrag_tr(const E* hi, const E* lo, int pitch, int k, int col0) {
    const int j = threadIdx.x & 15;
    const int off = (k + (j >> 2)) * pitch + col0 + 4 * (j & 3);
    SFrag<E> f;
    f.hi = __builtin_shufflevector(lds_tr16(hi + off), lds_tr16(hi + off + 4 * pitch), 0, 1, 2, 3, 4, 5, 6, 7);
    f.lo = __builtin_shufflevector(lds_tr16(lo + off), lds_tr16(lo + off + 4 * pitch), 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
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
