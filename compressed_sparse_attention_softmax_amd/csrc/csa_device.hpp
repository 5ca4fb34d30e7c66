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

// Accumulating MFMA with the accumulator pinned to the AGPR file ("+a"): a
// loop-carried accumulator then never moves between register files.  The
// compiler's hazard checks do not look inside inline asm, so every asm block
// below is self-contained: it opens with s_nop 1 (the 2 wait states an MFMA
// needs after a VALU or v_accvgpr write of any of its sources) and closes
// with CSA_MFMA_TAIL, 10 wait states: more than any read or write of a
// v_mfma_f32_16x16x32_bf16 result needs on gfx950 (a 4-pass XDL op; the
// compiler itself separates such a result from a VALU read by 8).  Whatever
// the register allocator places after a block -- a copy of an accumulator, a
// spill, a phi move at a loop exit -- therefore sees settled registers.
// Back-to-back accumulation into the same registers inside a block needs no
// wait states.  Blocks hold up to 8 MFMAs so that the tails cost little.
#define CSA_MFMA_TAIL "\n\ts_nop 9"
__device__ __forceinline__ void mfma16_acc(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b)
{
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" CSA_MFMA_TAIL : "+a"(acc) : "v"(a.v), "v"(b.v));
}
__device__ __forceinline__ void mfma16_acc(f32x4& acc, const Frag<float>& a, const Frag<float>& b)
{
    acc = mfma16(a, b, acc);
}
// Eight accumulating MFMAs in one asm block (one set of wait states):
// c_r += pa[r] * b0, then c_r += sa[r] * b1, r = 0..3; consecutive MFMAs use
// different accumulators.
__device__ __forceinline__ void mfma16x8_acc(f32x4& c0, f32x4& c1, f32x4& c2, f32x4& c3, const Frag<bf16_t>* pa,
                                             const Frag<bf16_t>* sa, const Frag<bf16_t>& b0, const Frag<bf16_t>& b1)
{
    asm("s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %12, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %5, %12, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %6, %12, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %7, %12, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %8, %13, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %10, %13, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %11, %13, %3" CSA_MFMA_TAIL
        : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
        : "v"(pa[0].v), "v"(pa[1].v), "v"(pa[2].v), "v"(pa[3].v), "v"(sa[0].v), "v"(sa[1].v), "v"(sa[2].v),
          "v"(sa[3].v), "v"(b0.v), "v"(b1.v));
}

// Four accumulating MFMAs in one asm block: c_r += pa[r] * b0, then
// c_r += sa[r] * b1, r = 0..1.
__device__ __forceinline__ void mfma16x4_acc(f32x4& c0, f32x4& c1, const Frag<bf16_t>* pa, const Frag<bf16_t>* sa,
                                             const Frag<bf16_t>& b0, const Frag<bf16_t>& b1)
{
    asm("s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %2, %6, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %3, %6, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %7, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %5, %7, %1" CSA_MFMA_TAIL
        : "+a"(c0), "+a"(c1)
        : "v"(pa[0].v), "v"(pa[1].v), "v"(sa[0].v), "v"(sa[1].v), "v"(b0.v), "v"(b1.v));
}

// Eight accumulating MFMAs: c_rj += pa[r] * b0[j], then c_rj += sa[r] * b1[j],
// r, j = 0..1 (two row tiles x two column tiles of a product pair).
__device__ __forceinline__ void mfma16_2x2_acc(f32x4& c00, f32x4& c01, f32x4& c10, f32x4& c11, const Frag<bf16_t>* pa,
                                               const Frag<bf16_t>* sa, const Frag<bf16_t>* b0, const Frag<bf16_t>* b1)
{
    asm("s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %8, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %5, %8, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %4, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %5, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %6, %10, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %7, %10, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %6, %11, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %7, %11, %3" CSA_MFMA_TAIL
        : "+a"(c00), "+a"(c01), "+a"(c10), "+a"(c11)
        : "v"(pa[0].v), "v"(pa[1].v), "v"(sa[0].v), "v"(sa[1].v), "v"(b0[0].v), "v"(b0[1].v), "v"(b1[0].v),
          "v"(b1[1].v));
}

// Eight accumulating MFMAs: c_j += pa * b0[j], then c_j += sa * b1[j], j = 0..3
// (one row tile x four column tiles of a product pair).
__device__ __forceinline__ void mfma16_1x4_acc(f32x4* c, const Frag<bf16_t>& pa, const Frag<bf16_t>& sa,
                                               const Frag<bf16_t>* b0, const Frag<bf16_t>* b1)
{
    asm("s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %4, %8, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %4, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %5, %10, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %5, %11, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %5, %12, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %5, %13, %3" CSA_MFMA_TAIL
        : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3])
        : "v"(pa.v), "v"(sa.v), "v"(b0[0].v), "v"(b0[1].v), "v"(b0[2].v), "v"(b0[3].v), "v"(b1[0].v), "v"(b1[1].v),
          "v"(b1[2].v), "v"(b1[3].v));
}

// Four independent accumulating MFMAs: c_j += a[j] * b[j], j = 0..3.
__device__ __forceinline__ void mfma16_4_acc(f32x4* c, const Frag<bf16_t>* a, const Frag<bf16_t>* b)
{
    asm("s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %8, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %5, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %6, %10, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %7, %11, %3" CSA_MFMA_TAIL
        : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3])
        : "v"(a[0].v), "v"(a[1].v), "v"(a[2].v), "v"(a[3].v), "v"(b[0].v), "v"(b[1].v), "v"(b[2].v), "v"(b[3].v));
}

// The two logit products of one row tile against four k steps, S += qa * r
// and dP += da * r, accumulating in VGPRs, with the row fragments r read
// from the AGPR file (an MFMA source may be either file): rows that stay
// resident for a whole kernel then hold no VGPRs.
__device__ __forceinline__ void mfma16_sd4_arows(f32x4& s, f32x4& d, const Frag<bf16_t>* qa, const Frag<bf16_t>* da,
                                                 const Frag<bf16_t>* r)
{
    asm("s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %2, %10, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %6, %10, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %3, %11, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %7, %11, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %4, %12, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %12, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1" CSA_MFMA_TAIL
        : "+v"(s), "+v"(d)
        : "v"(qa[0].v), "v"(qa[1].v), "v"(qa[2].v), "v"(qa[3].v), "v"(da[0].v), "v"(da[1].v), "v"(da[2].v),
          "v"(da[3].v), "a"(r[0].v), "a"(r[1].v), "a"(r[2].v), "a"(r[3].v));
}

// Zero accumulator created in the AGPR file (an MFMA of zero operands), so
// that a loop-carried accumulator is an AGPR value from its first definition.
// The trailing 32 wait states let the compiler copy the result right away.
__device__ __forceinline__ f32x4 agpr_zero()
{
    f32x4 acc;
    const bf16x8 z = {};
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0\n\ts_nop 15\n\ts_nop 15" : "=a"(acc) : "v"(z));
    return acc;
}

// Ordering point after the last mfma16_acc on accumulators a[0..N): the asm
// reads and writes all N, so no later use moves above it (the blocks are
// already settled by their own MFMA_TAIL; the extra wait states are kept).
template <int N> __device__ __forceinline__ void agpr_drain(f32x4* a);
template <> __device__ __forceinline__ void agpr_drain<8>(f32x4* a)
{
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]), "+a"(a[6]), "+a"(a[7]));
}
template <> __device__ __forceinline__ void agpr_drain<16>(f32x4* a)
{
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]), "+a"(a[6]), "+a"(a[7]), "+a"(a[8]), "+a"(a[9]), "+a"(a[10]), "+a"(a[11]), "+a"(a[12]), "+a"(a[13]), "+a"(a[14]), "+a"(a[15]));
}
template <> __device__ __forceinline__ void agpr_drain<32>(f32x4* a)
{
    asm volatile("s_nop 15\n\ts_nop 15" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]), "+a"(a[6]), "+a"(a[7]), "+a"(a[8]), "+a"(a[9]), "+a"(a[10]), "+a"(a[11]), "+a"(a[12]), "+a"(a[13]), "+a"(a[14]), "+a"(a[15]), "+a"(a[16]), "+a"(a[17]), "+a"(a[18]), "+a"(a[19]), "+a"(a[20]), "+a"(a[21]), "+a"(a[22]), "+a"(a[23]), "+a"(a[24]), "+a"(a[25]), "+a"(a[26]), "+a"(a[27]), "+a"(a[28]), "+a"(a[29]), "+a"(a[30]), "+a"(a[31]));
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

// Sums / maxima over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap moves: v_permlane16_swap exchanges odd and
// even rows between its two operands, v_permlane32_swap the two halves, so
// combining both results of each swap reduces across rows without LDS.
__device__ __forceinline__ float rows_sum(float v)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float v)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// 2^x on the transcendental unit (v_exp_f32): one instruction; results
// below 2^-126 flush to zero, which is harmless for softmax weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ------------------------------------------------------------ LDS tiles
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte words addressed by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Row-dependent permutation of the 8-element units of an LDS row: unit u of
// row r is stored at u ^ unit_swz(r, units).  Within any 16 consecutive rows
// (aligned) the XOR values are all different, so 16 lanes reading the same
// unit of 16 rows hit 16 different bank groups; within any 8 consecutive
// rows (aligned) they differ in more than the lowest bit, so 32 lanes reading
// a unit pair {2m, 2m+1} of 8 rows (the transposing read) hit 16 different
// bank groups.  `units` (a power of two) is the number of units per row.
__device__ __forceinline__ int unit_swz(int r, int units)
{
    return (((r & 7) << 1) | ((r >> 3) & 1)) & (units - 1);
}

// MFMA operand whose k index runs over rows of a row-major LDS tile:
// lane (n = lane%16, g = lane/16) gets column col0 + n of rows
// r0 + 4g + e (e = 0..3) and r0 + 16 + 4g + (e-4) (e = 4..7).
// This is the row order in which a 16x16 C tile pair (rows 0-15, 16-31 of a
// 32-row chunk, lane holding rows 4g+i) feeds the k slots of one operand.
// `stride` is the row stride in elements; with `swz` the tile is stored with
// 8-element units permuted per row (unit u of row r at u ^ unit_swz(r)).
template <typename T>
__device__ __forceinline__ Frag<T> rows_operand(const T* tile, int stride, int r0, int col0, bool swz)
{
    const int lane = lane_id(), g = lane / 16, n16 = lane % 16;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        const int r = r0 + 4 * g + (n16 >> 2);
        const int c = col0 + 4 * (n16 & 3);
        auto addr = [&](int rr) {
            const int cc = swz ? ((((c >> 3) ^ unit_swz(rr, stride >> 3)) << 3) | (c & 7)) : c;
            return tile + rr * stride + cc;
        };
        const bf16x4 a = ds_read_tr(addr(r));
        const bf16x4 b = ds_read_tr(addr(r + 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int rr = r0 + 16 * (e / 4) + 4 * g + (e % 4);
            const int c = col0 + n16;
            const int cc = swz ? ((((c >> 3) ^ unit_swz(rr, stride >> 3)) << 3) | (c & 7)) : c;
            f.v[e] = tile[rr * stride + cc];
        }
    }
    return f;
}

}  // namespace csa
