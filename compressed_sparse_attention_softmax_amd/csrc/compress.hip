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
#include "timing.hpp"

namespace csa {

namespace {

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

// Backward.  With alpha the pooling weights of block j, for a row u of its span
//   dx[u, c] += alpha dc[j, c],   dz[u, c] += alpha dc[j, c] (x[u, c] - c32[j, c]).
// A workgroup owns JB consecutive blocks and writes the rows u in
// [j0*ratio, (j0+JB)*ratio) exclusively (no atomics): it first recomputes the
// softmax state (max, 1/den, c32) and stages dc for every block whose span
// reaches those rows -- its own blocks plus the halo of later blocks when
// spans overlap -- then each thread gathers, for a (row, 8 channels) pair,
// the contributions of the blocks covering the row.  Rows past n_c*ratio are
// covered by no block and get zeros.
template <typename T, int D>
__global__ __launch_bounds__(256) void compress_bwd_kernel(const T* __restrict__ x,
                                                           const T* __restrict__ z, int zc,
                                                           const float* __restrict__ dc,
                                                           float* __restrict__ dx,
                                                           float* __restrict__ dz, int S, int r,
                                                           int L, int nc, int JB)
{
    constexpr int NCH = PoolState<T, D>::NCH;
    __shared__ float lds[3 * 256 * 8];
    extern __shared__ float st[];             // [block][4][D]: max, 1/den, c32, dc
    const int bi = blockIdx.y;
    const int j0 = blockIdx.x * JB;
    const int halo = (L + r - 1) / r - 1;
    const int jhi = min(nc, j0 + JB + halo);
    const int q = threadIdx.x % NCH, sp = threadIdx.x / NCH;
    const int64_t rowbase = (int64_t)bi * S;
    for (int j = j0; j < jhi; ++j) {
        const int hi = (j + 1) * r, lo = max(0, hi - L);
        float m[8], s[8], a[8];
        pool_block<T, D>(x, z, zc, rowbase, lo, hi, q, sp, m, s, a, lds);
        if (sp == 0) {
            float* sj = st + (size_t)(j - j0) * 4 * D;
            const Frag<float> gf = load_frag(dc + ((int64_t)bi * nc + j) * D + 8 * q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sj[8 * q + e] = m[e];
                sj[D + 8 * q + e] = 1.f / s[e];
                sj[2 * D + 8 * q + e] = a[e] / s[e];
                sj[3 * D + 8 * q + e] = gf.v[e];
            }
        }
        __syncthreads();     // the pooling scratch is reused by the next block
    }
    const int u_lo = j0 * r, u_hi = min(j0 + JB, nc) * r;
    const int npairs = (u_hi - u_lo) * NCH;
    const int nloop = (npairs + 255) / 256 * 256;     // whole waves stay together for the row sums
    for (int pr = threadIdx.x; pr < nloop; pr += 256) {
        const bool live = pr < npairs;
        const int u = u_lo + (live ? pr / NCH : 0);
        const int qq = pr % NCH;
        float xv[8], zv[8], gx[8], gz[8];
        float gzs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { gx[e] = 0.f; gz[e] = 0.f; }
        if (live) {
            load8(x + (rowbase + u) * D + 8 * qq, xv);
            if (zc == 1) {
                const float zz = to_f32(z[rowbase + u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) zv[e] = zz;
            } else {
                load8(z + (rowbase + u) * D + 8 * qq, zv);
            }
            const int jlast = min(nc - 1, (u + L) / r - 1);
            for (int j = u / r; j <= jlast; ++j) {
                const float* sj = st + (size_t)(j - j0) * 4 * D + 8 * qq;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ag = expf(zv[e] - sj[e]) * sj[D + e] * sj[3 * D + e];
                    gx[e] += ag;
                    gz[e] += ag * (xv[e] - sj[2 * D + e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) gzs += gz[e];
            Frag<float> fx;
#pragma unroll
            for (int e = 0; e < 8; ++e) fx.v[e] = gx[e];
            store_frag(dx + (rowbase + u) * D + 8 * qq, fx);
            if (zc != 1) {
                Frag<float> fz;
#pragma unroll
                for (int e = 0; e < 8; ++e) fz.v[e] = gz[e];
                store_frag(dz + (rowbase + u) * D + 8 * qq, fz);
            }
        }
        if (zc == 1) {
            // the NCH threads of a row are consecutive lanes of one wave
#pragma unroll
            for (int o = 1; o < NCH; o <<= 1) gzs += __shfl_xor(gzs, o);
            if (live && qq == 0) dz[rowbase + u] = gzs;
        }
    }
    // rows past the last block: no block covers them
    if (j0 + JB >= nc) {
        for (int i = threadIdx.x; i < (S - nc * r) * D; i += 256) dx[(rowbase + nc * r) * D + i] = 0.f;
        for (int i = threadIdx.x; i < (S - nc * r) * zc; i += 256) dz[(rowbase + nc * r) * zc + i] = 0.f;
    }
}

template <typename T, int D>
hipError_t launch_compress_fwd(const CompressArgs& p, hipStream_t st)
{
    dim3 grid(p.nc, p.b);
    TimedLaunch tl(K_COMPRESS_FWD, st);
    hipLaunchKernelGGL((compress_fwd_kernel<T, D>), grid, dim3(256), 0, st,
                       (const T*)p.x, (const T*)p.z, p.zc, (T*)p.c, p.c32, p.S, p.r, p.L, p.nc);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_compress_bwd(const CompressArgs& p, hipStream_t st)
{
    // about 512 workgroups, at most 16 blocks each
    int jb = (int)(((int64_t)p.nc * p.b) / 512);
    jb = jb < 1 ? 1 : (jb > 16 ? 16 : jb);
    const int halo = (p.L + p.r - 1) / p.r - 1;
    const size_t lds = (size_t)(jb + halo) * 4 * D * sizeof(float);
    auto kern = compress_bwd_kernel<T, D>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((p.nc + jb - 1) / jb, p.b);
    TimedLaunch tl(K_COMPRESS_BWD, st);
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, (const T*)p.x, (const T*)p.z, p.zc, p.dc, p.dx,
                       p.dz, p.S, p.r, p.L, p.nc, jb);
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
    if (p.nc == 0) {     // no block: every gradient row is zero
        hipError_t e = zero_fill(p.dx, (size_t)p.b * p.S * p.D, st);
        return e != hipSuccess ? e : zero_fill(p.dz, (size_t)p.b * p.S * p.zc, st);
    }
    switch (p.D) {
    case 64: return bf16 ? launch_compress_bwd<bf16_t, 64>(p, st) : launch_compress_bwd<float, 64>(p, st);
    case 128: return bf16 ? launch_compress_bwd<bf16_t, 128>(p, st) : launch_compress_bwd<float, 128>(p, st);
    case 512: return bf16 ? launch_compress_bwd<bf16_t, 512>(p, st) : launch_compress_bwd<float, 512>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csa
