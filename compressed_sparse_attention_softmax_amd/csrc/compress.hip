// compress.hip -- compressor softmax pooling, forward and backward (gfx950).
//
// Megatron-LM PR #6400, review thread on the compressor's pooling weights:
// softmax over the rows of a block in fp32, fp32 weighted sum, one cast of
// the pooled row to the working dtype.  Block j pools the rows
// [(j+1)*ratio - span, (j+1)*ratio) clipped at 0, channel by channel
// (z_channels == d) or with one score per row (z_channels == 1).
//
// HBM-bound: every element of x and z is read once (twice when spans
// overlap).  One workgroup of 256 threads owns block (b, j): the d channels
// are split in chunks of 8 (one 16-byte load per row for bf16) and the rows of
// the span are split over the remaining threads, each keeping an online
// softmax (running max, denominator, weighted sum) per channel; the partial
// states are merged through LDS.
#include "csa_device.hpp"
#include "csa_kernels.hpp"

namespace csa {

namespace {

template <typename T> struct Vec8 { float v[8]; };

template <typename T> __device__ __forceinline__ void load8(const T* p, float* out)
{
    Frag<T> f = load_frag(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = to_f32(f.v[e]);
}

template <typename T, int D>
struct PoolState {
    static constexpr int NCH = D / 8;
    static constexpr int NSPLIT = 256 / NCH;
};

// Per-thread online softmax over its share of the span's rows, then a merge
// over the row splits.  On return the threads with split 0 hold the block's
// (max, denominator, weighted sum) for their 8 channels.
template <typename T, int D>
__device__ __forceinline__ void pool_block(const T* __restrict__ x, const T* __restrict__ z,
                                           int zc, int64_t rowbase, int lo, int hi, int q, int sp,
                                           float* m, float* s, float* a, float* lds)
{
    constexpr int NCH = PoolState<T, D>::NCH;
    constexpr int NSPLIT = PoolState<T, D>::NSPLIT;
#pragma unroll
    for (int e = 0; e < 8; ++e) { m[e] = -INFINITY; s[e] = 0.f; a[e] = 0.f; }
    for (int u = lo + sp; u < hi; u += NSPLIT) {
        float xv[8], zv[8];
        load8(x + (rowbase + u) * D + 8 * q, xv);
        if (zc == 1) {
            float zz = to_f32(z[rowbase + u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) zv[e] = zz;
        } else {
            load8(z + (rowbase + u) * D + 8 * q, zv);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (zv[e] > m[e]) {
                float f = expf(m[e] - zv[e]);
                s[e] = s[e] * f + 1.f;
                a[e] = a[e] * f + xv[e];
                m[e] = zv[e];
            } else {
                float f = expf(zv[e] - m[e]);
                s[e] += f;
                a[e] += f * xv[e];
            }
        }
    }
    // merge the row splits: lds holds [3][256][8] floats
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lds[(0 * 256 + tid) * 8 + e] = m[e];
        lds[(1 * 256 + tid) * 8 + e] = s[e];
        lds[(2 * 256 + tid) * 8 + e] = a[e];
    }
    __syncthreads();
    if (sp == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float M = -INFINITY;
            for (int k = 0; k < NSPLIT; ++k) M = fmaxf(M, lds[(0 * 256 + k * NCH + q) * 8 + e]);
            float S = 0.f, A = 0.f;
            for (int k = 0; k < NSPLIT; ++k) {
                float mk = lds[(0 * 256 + k * NCH + q) * 8 + e];
                float f = mk == -INFINITY ? 0.f : expf(mk - M);
                S += lds[(1 * 256 + k * NCH + q) * 8 + e] * f;
                A += lds[(2 * 256 + k * NCH + q) * 8 + e] * f;
            }
            m[e] = M; s[e] = S; a[e] = A;
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void compress_fwd_kernel(const T* __restrict__ x,
                                                           const T* __restrict__ z, int zc,
                                                           T* __restrict__ c, float* __restrict__ c32,
                                                           int S, int r, int L, int nc)
{
    constexpr int NCH = PoolState<T, D>::NCH;
    __shared__ float lds[3 * 256 * 8];
    const int j = blockIdx.x, bi = blockIdx.y;
    const int q = threadIdx.x % NCH, sp = threadIdx.x / NCH;
    const int hi = (j + 1) * r, lo = max(0, hi - L);
    float m[8], s[8], a[8];
    pool_block<T, D>(x, z, zc, (int64_t)bi * S, lo, hi, q, sp, m, s, a, lds);
    if (sp == 0) {
        const int64_t o = ((int64_t)bi * nc + j) * D + 8 * q;
        Frag<T> f;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { v[e] = a[e] / s[e]; f.v[e] = from_f32<T>(v[e]); }
        store_frag(c + o, f);
        if (c32) {
            Frag<float> g;
#pragma unroll
            for (int e = 0; e < 8; ++e) g.v[e] = v[e];
            store_frag(c32 + o, g);
        }
    }
}

// Backward: recompute the block's softmax state, then for every row of the
// span  alpha = exp(z - max) / den,  dx += alpha dc,  dz += alpha dc (x - c32).
// Spans that overlap (span > ratio) share rows with the neighbouring block, so
// those rows are accumulated with fp32 atomics; otherwise each row belongs to
// exactly one block and is stored directly.  dx and dz arrive zero-filled.
template <typename T, int D>
__global__ __launch_bounds__(256) void compress_bwd_kernel(const T* __restrict__ x,
                                                           const T* __restrict__ z, int zc,
                                                           const float* __restrict__ dc,
                                                           float* __restrict__ dx,
                                                           float* __restrict__ dz, int S, int r,
                                                           int L, int nc)
{
    constexpr int NCH = PoolState<T, D>::NCH;
    constexpr int NSPLIT = PoolState<T, D>::NSPLIT;
    __shared__ float lds[3 * 256 * 8];
    __shared__ float fin[3][D];
    const int j = blockIdx.x, bi = blockIdx.y;
    const int q = threadIdx.x % NCH, sp = threadIdx.x / NCH;
    const int hi = (j + 1) * r, lo = max(0, hi - L);
    const int64_t rowbase = (int64_t)bi * S;
    float m[8], s[8], a[8];
    pool_block<T, D>(x, z, zc, rowbase, lo, hi, q, sp, m, s, a, lds);
    if (sp == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            fin[0][8 * q + e] = m[e];
            fin[1][8 * q + e] = 1.f / s[e];
            fin[2][8 * q + e] = a[e] / s[e];
        }
    }
    __syncthreads();
    float M[8], IS[8], C32[8], G[8];
    Frag<float> gf = load_frag(dc + ((int64_t)bi * nc + j) * D + 8 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        M[e] = fin[0][8 * q + e]; IS[e] = fin[1][8 * q + e]; C32[e] = fin[2][8 * q + e];
        G[e] = gf.v[e];
    }
    const bool exclusive = L <= r;
    for (int u = lo + sp; u < hi; u += NSPLIT) {
        float xv[8], zv[8];
        load8(x + (rowbase + u) * D + 8 * q, xv);
        if (zc == 1) {
            float zz = to_f32(z[rowbase + u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) zv[e] = zz;
        } else {
            load8(z + (rowbase + u) * D + 8 * q, zv);
        }
        float gx[8], gz[8], gzs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float alpha = expf(zv[e] - M[e]) * IS[e];
            gx[e] = alpha * G[e];
            gz[e] = gx[e] * (xv[e] - C32[e]);
            gzs += gz[e];
        }
        float* px = dx + (rowbase + u) * D + 8 * q;
        if (exclusive) {
            Frag<float> f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f.v[e] = gx[e];
            store_frag(px, f);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) atomicAdd(px + e, gx[e]);
        }
        if (zc == 1) {
            atomicAdd(dz + rowbase + u, gzs);
        } else {
            float* pz = dz + (rowbase + u) * D + 8 * q;
            if (exclusive) {
                Frag<float> f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f.v[e] = gz[e];
                store_frag(pz, f);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) atomicAdd(pz + e, gz[e]);
            }
        }
    }
}

template <typename T, int D>
hipError_t launch_compress_fwd(const CompressArgs& p, hipStream_t st)
{
    dim3 grid(p.nc, p.b);
    hipLaunchKernelGGL((compress_fwd_kernel<T, D>), grid, dim3(256), 0, st,
                       (const T*)p.x, (const T*)p.z, p.zc, (T*)p.c, p.c32, p.S, p.r, p.L, p.nc);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_compress_bwd(const CompressArgs& p, hipStream_t st)
{
    dim3 grid(p.nc, p.b);
    hipLaunchKernelGGL((compress_bwd_kernel<T, D>), grid, dim3(256), 0, st,
                       (const T*)p.x, (const T*)p.z, p.zc, p.dc, p.dx, p.dz, p.S, p.r, p.L, p.nc);
    return hipGetLastError();
}

}  // namespace

hipError_t compress_fwd(const CompressArgs& p, bool bf16, hipStream_t st)
{
    if (p.nc == 0) return hipSuccess;
    switch (p.D) {
    case 64: return bf16 ? launch_compress_fwd<bf16_t, 64>(p, st) : launch_compress_fwd<float, 64>(p, st);
    case 128: return bf16 ? launch_compress_fwd<bf16_t, 128>(p, st) : launch_compress_fwd<float, 128>(p, st);
    case 512: return bf16 ? launch_compress_fwd<bf16_t, 512>(p, st) : launch_compress_fwd<float, 512>(p, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t compress_bwd(const CompressArgs& p, bool bf16, hipStream_t st)
{
    if (p.nc == 0) return hipSuccess;
    switch (p.D) {
    case 64: return bf16 ? launch_compress_bwd<bf16_t, 64>(p, st) : launch_compress_bwd<float, 64>(p, st);
    case 128: return bf16 ? launch_compress_bwd<bf16_t, 128>(p, st) : launch_compress_bwd<float, 128>(p, st);
    case 512: return bf16 ? launch_compress_bwd<bf16_t, 512>(p, st) : launch_compress_bwd<float, 512>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csa
