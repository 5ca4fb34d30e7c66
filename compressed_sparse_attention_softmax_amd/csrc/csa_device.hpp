// csa_device.hpp -- device helpers for the gfx950 (CDNA4) CSA kernels.
//
// Matrix-core tiles are v_mfma_f32_16x16x32_bf16 (fp32 inputs: eight
// v_mfma_f32_16x16x4_f32 steps).  Lane layout of one 16x16x32 step on a
// 64-lane wave, with g = lane / 16 and n = lane % 16:
//   A (16 x 32): lane holds A[m = n][k = 8g + e],  e = 0..7
//   B (32 x 16): lane holds B[k = 8g + e][n]
//   C (16 x 16): lane holds C[m = 4g + i][n],       i = 0..3
// Every contraction below loads A and B with the same k <-> lane map, so any
// relabelling of k is harmless; where a C tile is reused as an operand the
// mapping of its rows onto k is spelled out at the use.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

template <typename T> struct Frag;
template <> struct Frag<bf16_t> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ f32x4 mfma16(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const Frag<float>& a, const Frag<float>& b, f32x4 c)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
}

template <typename T> __device__ __forceinline__ Frag<T> zero_frag()
{
    Frag<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (T)0.0f;
    return f;
}

// 8 consecutive elements (16 B for bf16, 32 B for fp32)
__device__ __forceinline__ Frag<bf16_t> load_frag(const bf16_t* p)
{
    Frag<bf16_t> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
}
__device__ __forceinline__ Frag<float> load_frag(const float* p)
{
    Frag<float> f;
    f.v = *reinterpret_cast<const f32x8*>(p);
    return f;
}
__device__ __forceinline__ void store_frag(bf16_t* p, const Frag<bf16_t>& f)
{
    *reinterpret_cast<bf16x8*>(p) = f.v;
}
__device__ __forceinline__ void store_frag(float* p, const Frag<float>& f)
{
    *reinterpret_cast<f32x8*>(p) = f.v;
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

__device__ __forceinline__ f32x4 f4zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__device__ __forceinline__ unsigned mbcnt(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// 2^x on the transcendental unit (v_exp_f32): one instruction; results
// below 2^-126 flush to zero, which is harmless for softmax weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

}  // namespace csa
