// Device-side helpers shared by the kernel sources: operand fragments and
// their conversions, the matrix instruction, SiLU's sigmoid, the fused
// momentum / forgetting write and token addressing.  Not part of the public
// interface.
#pragma once

#include "tm_internal.h"

namespace tmk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <class OP> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 T; };
template <> struct Frag<float> { typedef f32x8 T; };   // also: 8 raw values of a storage type

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ f32x8 ld8(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
// 8 consecutive outputs of one input of W_1's accumulator-order master
__device__ __forceinline__ f32x8 ld8w1(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 64);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 to_bf16(f32x8 v) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)v[j];
    return r;
}
__device__ __forceinline__ f32x8 to_f32(bf16x8 v) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (float)v[j];
    return r;
}

template <class OP> __device__ __forceinline__ typename Frag<OP>::T cvt(f32x8 v);
template <> __device__ __forceinline__ bf16x8 cvt<bf16>(f32x8 v) { return to_bf16(v); }
template <> __device__ __forceinline__ f32x8 cvt<float>(f32x8 v) { return v; }
template <class OP> __device__ __forceinline__ typename Frag<OP>::T cvt(bf16x8 v);
template <> __device__ __forceinline__ bf16x8 cvt<bf16>(bf16x8 v) { return v; }
template <> __device__ __forceinline__ f32x8 cvt<float>(bf16x8 v) { return to_f32(v); }

__device__ __forceinline__ f32x8 to_f32v(f32x8 v) { return v; }
__device__ __forceinline__ f32x8 to_f32v(bf16x8 v) { return to_f32(v); }

template <class OP> __device__ __forceinline__ typename Frag<OP>::T zero_frag() {
    typename Frag<OP>::T z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (OP)0.0f;
    return z;
}

// v where `on`, else zeros, by a bit mask the optimizer cannot see through:
// written as `on ? v : 0`, the load behind v is moved into a branch on `on`
// and issued late, behind a wait for every load before it.
template <class F> __device__ __forceinline__ F keep_if(F v, bool on) {
    typedef int IV __attribute__((ext_vector_type(sizeof(F) / 4)));
    int m = on ? -1 : 0;
    asm volatile("" : "+v"(m));
    return __builtin_bit_cast(F, __builtin_bit_cast(IV, v) & m);
}

// C += A B over one 32-deep slice of K.  Each lane supplies 8 consecutive K
// values of its A row and of its B column; A and B use the same K order, so
// how the instruction maps register slots to K does not matter.
__device__ __forceinline__ void mma(f32x4& c, bf16x8 a, bf16x8 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, f32x8 a, f32x8 b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}

// sigma(z) = 1 / (1 + e^-z) with the hardware exponential and reciprocal
// (each about 1 ulp): saturates to 0 and 1, propagates NaN
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// The new M and S of a chunk (one float4 of the accumulator-order layout).
// Plain stores: measured against non-temporal and write-through (sc1)
// stores, which both made the chunk step slower.
__device__ __forceinline__ void st_state(float* p, f32x4 v) {
    *reinterpret_cast<f32x4*>(p) = v;
}

// The chunk's momentum / forgetting write of one element, with explicit
// fused multiply-adds, so that every kernel (and every instantiation of one)
// rounds it the same way:  S' = p_eta S - U_S,  M' = p_alpha M + s0 S - U_M.
__device__ __forceinline__ float mom_s(float pe, float s, float us) { return __builtin_fmaf(pe, s, -us); }
__device__ __forceinline__ float mom_m(float pa, float m, float s0, float s, float um) {
    return __builtin_fmaf(pa, m, __builtin_fmaf(s0, s, -um));
}

__device__ __forceinline__ long tok_off(const TokLayout& tl, int s, int t) {
    int bi = s / tl.H, hi = s - bi * tl.H;
    return ((long)bi * tl.Tc + t) * tl.H * (long)tl.d + (long)hi * tl.d;
}

template <class T> __device__ __forceinline__ void store1(void* p, long i, float x) {
    reinterpret_cast<T*>(p)[i] = (T)x;
}
template <class T> __device__ __forceinline__ float load1(const void* p, long i) {
    return (float)reinterpret_cast<const T*>(p)[i];
}

}  // namespace tmk
