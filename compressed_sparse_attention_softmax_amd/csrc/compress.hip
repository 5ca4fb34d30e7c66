// compress.hip -- compressor softmax pooling, forward and backward (gfx950).
//
// Megatron-LM PR #6400, review thread on the compressor's pooling weights:
// softmax over the rows of a block in fp32, fp32 weighted sum, one cast of
// the pooled row to the working dtype.  Block j pools the rows
// [(j+1)*ratio - span, (j+1)*ratio) clipped at 0, channel by channel
// (z_channels == d) or with one score per row (z_channels == 1).
//
// HBM-bound: every element of x and z is read once (twice when spans
// overlap).  A group of NS consecutive lanes owns one (block, 8 channels)
// pair: lane split sp takes the span rows lo + sp, lo + sp + NS, ... in groups
// of 8 (one 16-byte load per row for bf16), keeping a running max, denominator
// and weighted sum per channel, and the NS partial states are merged with
// lane shuffles.  NS never exceeds the ratio, so every split owns at least one
// row of every span (spans are clipped at 0 but keep at least `ratio` rows).
//
// Epilogue (same PR: the pooled row, cast once, goes through the
// compressor's norm; layer configuration thread: the compressed rows get a
// rotary embedding with base 40000): an RMS norm with a per-channel weight,
// then the last rope_dim channels of block j's row turned in interleaved
// pairs (2i, 2i+1) by the angle j * base^(-2i / rope_dim).  It runs in place
// on the cast rows, one group of D/8 consecutive lanes per row (the row sum
// by lane shuffles); angles are formed in fp64.  Its backward recomputes the
// pooled row, applies the transposed rotation and the norm's backward, and
// hands the gradient of the pooled rows to the pooling backward through the
// workspace; the weight gradient is summed per workgroup and then over
// workgroups, in a fixed order.
#include <algorithm>

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

// e^x on the transcendental unit (v_exp_f32 after a multiply by log2 e)
__device__ __forceinline__ float fexp(float x) { return fast_exp2(x * LOG2E); }

// element strides (batch, token) of x and dx, and of z and dz
struct RowStrides { int64_t xb, xs, zb, zs; };
RowStrides row_strides(const CompressArgs& p) { return RowStrides{p.xsb, p.xss, p.zsb, p.zss}; }

// Softmax state (max m, denominator s, weighted sum a) of the 8 channels
// [8q, 8q+8) over the rows [lo, hi) of one span, split NS ways over
// consecutive lanes; every lane of the group returns the merged state.  x and
// z point at the batch's first row; rows are xs and zs elements apart.
template <typename T, int D, int NS>
__device__ __forceinline__ void span_state(const T* __restrict__ x, int64_t xs, const T* __restrict__ z,
                                           int64_t zs, int zc, int lo, int hi, int q, int sp,
                                           float* m, float* s, float* a)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) { m[e] = -INFINITY; s[e] = 0.f; a[e] = 0.f; }
    for (int u0 = lo + sp; u0 < hi; u0 += 8 * NS) {
        float xv[8][8], zv[8][8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int u = u0 + k * NS;
            if (u < hi) {
                load8(x + u * xs + 8 * q, xv[k]);
                if (zc == 1) {
                    const float zz = to_f32(z[u * zs]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) zv[k][e] = zz;
                } else {
                    load8(z + u * zs + 8 * q, zv[k]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) { xv[k][e] = 0.f; zv[k][e] = -INFINITY; }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float gm = zv[0][e];
#pragma unroll
            for (int k = 1; k < 8; ++k) gm = fmaxf(gm, zv[k][e]);
            const float mn = fmaxf(m[e], gm);      // finite: the first group of a split has a row
            const float f = fexp(m[e] - mn);
            float ss = 0.f, aa = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float w = fexp(zv[k][e] - mn);
                ss += w;
                aa += w * xv[k][e];
            }
            s[e] = s[e] * f + ss;
            a[e] = a[e] * f + aa;
            m[e] = mn;
        }
    }
#pragma unroll
    for (int o = 1; o < NS; o <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float mo = __shfl_xor(m[e], o), so = __shfl_xor(s[e], o), ao = __shfl_xor(a[e], o);
            const float mn = fmaxf(m[e], mo);
            const float f0 = fexp(m[e] - mn), f1 = fexp(mo - mn);
            s[e] = s[e] * f0 + so * f1;
            a[e] = a[e] * f0 + ao * f1;
            m[e] = mn;
        }
    }
}

// one lane group per (batch, block, 8 channels)
template <typename T, int D, int NS>
__global__ __launch_bounds__(256) void compress_fwd_kernel(const T* __restrict__ x,
                                                           const T* __restrict__ z, int zc,
                                                           T* __restrict__ c, float* __restrict__ c32,
                                                           int b, int S, int r, int L, int nc, RowStrides rs)
{
    constexpr int NCH = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)b * nc * NCH * NS;
    const bool live = gid < total;                 // whole lane groups share liveness
    const int64_t gg = live ? gid : 0;
    const int sp = (int)(gg % NS);
    const int q = (int)(gg / NS % NCH);
    const int64_t bj = gg / NS / NCH;
    const int j = (int)(bj % nc), bi = (int)(bj / nc);
    const int hi = (j + 1) * r, lo = max(0, hi - L);
    float m[8], s[8], a[8];
    span_state<T, D, NS>(x + bi * rs.xb, rs.xs, z + bi * rs.zb, rs.zs, zc, lo, hi, q, sp, m, s, a);
    if (live && sp == 0) {
        const int64_t o = bj * D + 8 * q;
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

// --------------------------------------------------------------- epilogue
// cos / sin of pair i of block j's rotation (fp64 angle: j * base^(-2i/rope_dim))
__device__ __forceinline__ void rope_cs(int j, int i, int rope_dim, float base, float& cs, float& sn)
{
    const double ang = (double)j * pow((double)base, -2.0 * i / rope_dim);
    double s2, c2;
    sincos(ang, &s2, &c2);
    cs = (float)c2;
    sn = (float)s2;
}

// rotate (sign = 1) or rotate back (sign = -1) the pairs of channels
// [8q, 8q+8) that lie in the last rope_dim channels
template <int D>
__device__ __forceinline__ void rope8(float* v, int q, int j, int rope_dim, float base, float sign)
{
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
        const int ch = 8 * q + 2 * pr;
        if (ch >= D - rope_dim) {
            float cs, sn;
            rope_cs(j, (ch - (D - rope_dim)) / 2, rope_dim, base, cs, sn);
            sn *= sign;
            const float x0 = v[2 * pr], x1 = v[2 * pr + 1];
            v[2 * pr] = x0 * cs - x1 * sn;
            v[2 * pr + 1] = x0 * sn + x1 * cs;
        }
    }
}

// sum over the D/8 lanes of a row group (consecutive lanes of one wave)
template <int D>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int o = 1; o < D / 8; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// in place on the cast pooled rows c [rows, D]
template <typename T, int D>
__global__ __launch_bounds__(256) void compress_epi_fwd_kernel(T* __restrict__ c, const float* __restrict__ nw,
                                                               float eps, int rope_dim, float base, int64_t rows,
                                                               int nc)
{
    constexpr int G = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = gid < rows * G;             // whole groups share liveness
    const int64_t gg = live ? gid : 0;
    const int q = (int)(gg % G);
    const int64_t bj = gg / G;
    const int j = (int)(bj % nc);
    float v[8];
    load8(c + bj * D + 8 * q, v);
    if (nw) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        const float inv = rsqrtf(group_sum<D>(ss) / D + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * inv * nw[8 * q + e];
    }
    rope8<D>(v, q, j, rope_dim, base, 1.f);
    if (live) {
        Frag<T> f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = from_f32<T>(v[e]);
        store_frag(c + bj * D + 8 * q, f);
    }
}

// dy (gradient of the pooled rows) into the workspace; per-workgroup sums of
// the weight gradient into `wpart` [gridDim.x, D]
template <typename T, int D>
__global__ __launch_bounds__(256) void compress_epi_bwd_kernel(const T* __restrict__ x, const T* __restrict__ z,
                                                               int zc, const float* __restrict__ nw, float eps,
                                                               int rope_dim, float base,
                                                               const float* __restrict__ dc, float* __restrict__ dy,
                                                               float* __restrict__ wpart, int S, int r, int L,
                                                               int64_t rows, int nc, RowStrides rs)
{
    constexpr int G = D / 8, RPW = 256 / G;
    __shared__ float dws[RPW * D];
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = gid < rows * G;
    const int64_t gg = live ? gid : 0;
    const int q = (int)(gg % G);
    const int64_t bj = gg / G;
    const int j = (int)(bj % nc), bi = (int)(bj / nc);
    const int hi = (j + 1) * r, lo = max(0, hi - L);
    float m[8], s[8], a[8], y[8], g[8];
    span_state<T, D, 1>(x + bi * rs.xb, rs.xs, z + bi * rs.zb, rs.zs, zc, lo, hi, q, 0, m, s, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = to_f32(from_f32<T>(a[e] / s[e]));   // the cast pooled row
    const Frag<float> df = load_frag(dc + bj * D + 8 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = df.v[e];
    rope8<D>(g, q, j, rope_dim, base, -1.f);          // transpose of the rotation
    float out[8], dwv[8];
    if (nw) {
        float ss = 0.f, sg = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss += y[e] * y[e];
            sg += nw[8 * q + e] * g[e] * y[e];
        }
        ss = group_sum<D>(ss);
        sg = group_sum<D>(sg);
        const float inv = rsqrtf(ss / D + eps);
        const float k3 = inv * inv * inv * sg / D;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            out[e] = inv * nw[8 * q + e] * g[e] - k3 * y[e];
            dwv[e] = live ? g[e] * y[e] * inv : 0.f;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { out[e] = g[e]; dwv[e] = 0.f; }
    }
    if (live) {
        Frag<float> f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = out[e];
        store_frag(dy + bj * D + 8 * q, f);
    }
    if (wpart) {                                      // uniform over the workgroup
        // slot of this lane in the workgroup's rows (lanes past the last row
        // write their zeros to their own slot too)
        const int rw = (int)threadIdx.x / G, ql = (int)threadIdx.x % G;
#pragma unroll
        for (int e = 0; e < 8; ++e) dws[rw * D + 8 * ql + e] = dwv[e];
        __syncthreads();
        for (int ch = threadIdx.x; ch < D; ch += 256) {
            float acc = 0.f;
            for (int k = 0; k < RPW; ++k) acc += dws[k * D + ch];
            wpart[(int64_t)blockIdx.x * D + ch] = acc;
        }
    }
}

// weight gradient: sum of the per-workgroup parts in workgroup order
__global__ __launch_bounds__(256) void compress_epi_wsum_kernel(const float* __restrict__ wpart, int nparts, int D,
                                                                float* __restrict__ dnw)
{
    for (int ch = threadIdx.x; ch < D; ch += 256) {
        float acc = 0.f;
        for (int k = 0; k < nparts; ++k) acc += wpart[(int64_t)k * D + ch];
        dnw[ch] = acc;
    }
}

// Backward.  With alpha the pooling weights of block j, for a row u of its span
//   dx[u, c] += alpha dc[j, c],   dz[u, c] += alpha dc[j, c] (x[u, c] - c32[j, c]).
// A workgroup owns JB consecutive blocks and writes the rows u in
// [j0*ratio, (j0+JB)*ratio) exclusively (no atomics): it first recomputes the
// softmax state (max, 1/den, c32) and stages dc for every block whose span
// reaches those rows -- its own blocks plus the halo of later blocks when
// spans overlap -- all blocks at once, then each thread gathers, for a
// (row, 8 channels) pair, the contributions of the blocks covering the row.
// Rows past n_c*ratio are covered by no block and get zeros.
template <typename T, int D, int NS>
__global__ __launch_bounds__(256) void compress_bwd_kernel(const T* __restrict__ x,
                                                           const T* __restrict__ z, int zc,
                                                           const float* __restrict__ dc,
                                                           float* __restrict__ dx,
                                                           float* __restrict__ dz, int S, int r,
                                                           int L, int nc, int JB, RowStrides rs)
{
    constexpr int NCH = D / 8;
    extern __shared__ float st[];             // [block][4][D]: max, 1/den, c32, dc
    const int bi = blockIdx.y;
    const int j0 = blockIdx.x * JB;
    const int halo = (L + r - 1) / r - 1;
    const int jhi = min(nc, j0 + JB + halo);
    // the batch's first rows of x, z, dx and dz
    const T* xr = x + bi * rs.xb;
    const T* zr = z + bi * rs.zb;
    float* dxr = dx + bi * rs.xb;
    float* dzr = dz + bi * rs.zb;
    // softmax state of every block the workgroup needs, NS lanes per (block, chunk)
    const int nst = (jhi - j0) * NCH * NS;
    for (int i0 = 0; i0 < nst; i0 += 256) {       // uniform trip count: groups stay whole
        const int i = i0 + (int)threadIdx.x;
        const bool live = i < nst;
        const int ii = live ? i : 0;
        const int sp = ii % NS, q = ii / NS % NCH, j = j0 + ii / NS / NCH;
        const int hi = (j + 1) * r, lo = max(0, hi - L);
        float m[8], s[8], a[8];
        span_state<T, D, NS>(xr, rs.xs, zr, rs.zs, zc, lo, hi, q, sp, m, s, a);
        if (live && sp == 0) {
            float* sj = st + (size_t)(j - j0) * 4 * D;
            const Frag<float> gf = load_frag(dc + ((int64_t)bi * nc + j) * D + 8 * q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float inv = 1.f / s[e];
                sj[8 * q + e] = m[e];
                sj[D + 8 * q + e] = inv;
                sj[2 * D + 8 * q + e] = a[e] * inv;
                sj[3 * D + 8 * q + e] = gf.v[e];
            }
        }
    }
    __syncthreads();
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
            load8(xr + u * rs.xs + 8 * qq, xv);
            if (zc == 1) {
                const float zz = to_f32(zr[u * rs.zs]);
#pragma unroll
                for (int e = 0; e < 8; ++e) zv[e] = zz;
            } else {
                load8(zr + u * rs.zs + 8 * qq, zv);
            }
            const int jlast = min(nc - 1, (u + L) / r - 1);
            for (int j = u / r; j <= jlast; ++j) {
                const float* sj = st + (size_t)(j - j0) * 4 * D + 8 * qq;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ag = fexp(zv[e] - sj[e]) * sj[D + e] * sj[3 * D + e];
                    gx[e] += ag;
                    gz[e] += ag * (xv[e] - sj[2 * D + e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) gzs += gz[e];
            Frag<float> fx;
#pragma unroll
            for (int e = 0; e < 8; ++e) fx.v[e] = gx[e];
            store_frag(dxr + u * rs.xs + 8 * qq, fx);
            if (zc != 1) {
                Frag<float> fz;
#pragma unroll
                for (int e = 0; e < 8; ++e) fz.v[e] = gz[e];
                store_frag(dzr + u * rs.zs + 8 * qq, fz);
            }
        }
        if (zc == 1) {
            // the NCH threads of a row are consecutive lanes of one wave
#pragma unroll
            for (int o = 1; o < NCH; o <<= 1) gzs += __shfl_xor(gzs, o);
            if (live && qq == 0) dzr[u * rs.zs] = gzs;
        }
    }
    // rows past the last block: no block covers them
    if (j0 + JB >= nc) {
        for (int i = threadIdx.x; i < (S - nc * r) * D; i += 256) dxr[(nc * r + i / D) * rs.xs + i % D] = 0.f;
        for (int i = threadIdx.x; i < (S - nc * r) * zc; i += 256) dzr[(nc * r + i / zc) * rs.zs + i % zc] = 0.f;
    }
}

// lanes per span: a power of two, at most the ratio (every split keeps a row)
// and about one group of 8 rows per lane, at most 8
inline int span_splits(int r, int L)
{
    int ns = 1;
    while (ns * 2 <= 8 && ns * 2 <= r && ns * 2 * 8 <= L) ns *= 2;
    return ns;
}

template <typename T, int D, int NS>
hipError_t launch_compress_fwd_ns(const CompressArgs& p, hipStream_t st)
{
    const int64_t threads = (int64_t)p.b * p.nc * (D / 8) * NS;
    dim3 grid((unsigned)((threads + 255) / 256));
    TimedLaunch tl(K_COMPRESS_FWD, st);
    hipLaunchKernelGGL((compress_fwd_kernel<T, D, NS>), grid, dim3(256), 0, st, (const T*)p.x, (const T*)p.z, p.zc,
                       (T*)p.c, p.c32, p.b, p.S, p.r, p.L, p.nc, row_strides(p));
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_compress_fwd(const CompressArgs& p, hipStream_t st)
{
    switch (span_splits(p.r, p.L)) {
    case 1: return launch_compress_fwd_ns<T, D, 1>(p, st);
    case 2: return launch_compress_fwd_ns<T, D, 2>(p, st);
    case 4: return launch_compress_fwd_ns<T, D, 4>(p, st);
    default: return launch_compress_fwd_ns<T, D, 8>(p, st);
    }
}

template <typename T, int D, int NS>
hipError_t launch_compress_bwd_ns(const CompressArgs& p, hipStream_t st)
{
    // about 512 workgroups, at most 16 blocks each
    int jb = (int)(((int64_t)p.nc * p.b) / 512);
    jb = jb < 1 ? 1 : (jb > 16 ? 16 : jb);
    const int halo = (p.L + p.r - 1) / p.r - 1;
    const size_t lds = (size_t)(jb + halo) * 4 * D * sizeof(float);
    auto kern = compress_bwd_kernel<T, D, NS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((p.nc + jb - 1) / jb, p.b);
    TimedLaunch tl(K_COMPRESS_BWD, st);
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, (const T*)p.x, (const T*)p.z, p.zc, p.dc, p.dx,
                       p.dz, p.S, p.r, p.L, p.nc, jb, row_strides(p));
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_compress_bwd(const CompressArgs& p, hipStream_t st)
{
    switch (span_splits(p.r, p.L)) {
    case 1: return launch_compress_bwd_ns<T, D, 1>(p, st);
    case 2: return launch_compress_bwd_ns<T, D, 2>(p, st);
    case 4: return launch_compress_bwd_ns<T, D, 4>(p, st);
    default: return launch_compress_bwd_ns<T, D, 8>(p, st);
    }
}

bool has_epilogue(const CompressArgs& p) { return p.norm_w || p.rope_dim > 0; }

int64_t epi_parts(const CompressArgs& p) { return ((int64_t)p.b * p.nc * (p.D / 8) + 255) / 256; }

template <typename T, int D>
hipError_t launch_epi_fwd(const CompressArgs& p, hipStream_t st)
{
    const int64_t rows = (int64_t)p.b * p.nc;
    TimedLaunch tl(K_COMPRESS_EPI, st);
    hipLaunchKernelGGL((compress_epi_fwd_kernel<T, D>), dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0,
                       st, (T*)p.c, p.norm_w, p.eps, p.rope_dim, p.rope_base, rows, p.nc);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t compress_fwd_d(const CompressArgs& p, hipStream_t st)
{
    hipError_t e = launch_compress_fwd<T, D>(p, st);
    if (e != hipSuccess || !has_epilogue(p)) return e;
    return launch_epi_fwd<T, D>(p, st);
}

// epilogue backward: dy into the workspace, then the pooling backward from dy
template <typename T, int D>
hipError_t compress_bwd_d(const CompressArgs& p, hipStream_t st)
{
    if (!has_epilogue(p)) return launch_compress_bwd<T, D>(p, st);
    const int64_t rows = (int64_t)p.b * p.nc;
    const int64_t parts = epi_parts(p);
    float* dy = p.ws;
    float* wpart = p.dnorm_w ? p.ws + rows * D : nullptr;
    {
        TimedLaunch tl(K_COMPRESS_EPI, st);
        hipLaunchKernelGGL((compress_epi_bwd_kernel<T, D>), dim3((unsigned)parts), dim3(256), 0, st, (const T*)p.x,
                           (const T*)p.z, p.zc, p.norm_w, p.eps, p.rope_dim, p.rope_base, p.dc, dy, wpart, p.S, p.r,
                           p.L, rows, p.nc, row_strides(p));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (wpart) {
            hipLaunchKernelGGL(compress_epi_wsum_kernel, dim3(1), dim3(256), 0, st, wpart, (int)parts, D, p.dnorm_w);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    CompressArgs q = p;
    q.dc = dy;
    return launch_compress_bwd<T, D>(q, st);
}

}  // namespace

size_t compress_bwd_workspace_bytes(const CompressArgs& p)
{
    if (!has_epilogue(p) || p.nc == 0) return 0;
    return (size_t)((int64_t)p.b * p.nc * p.D + epi_parts(p) * p.D) * sizeof(float);
}

hipError_t compress_fwd(const CompressArgs& p, bool bf16, hipStream_t st)
{
    if (p.nc == 0) return hipSuccess;
    switch (p.D) {
    case 64: return bf16 ? compress_fwd_d<bf16_t, 64>(p, st) : compress_fwd_d<float, 64>(p, st);
    case 128: return bf16 ? compress_fwd_d<bf16_t, 128>(p, st) : compress_fwd_d<float, 128>(p, st);
    case 512: return bf16 ? compress_fwd_d<bf16_t, 512>(p, st) : compress_fwd_d<float, 512>(p, st);
    default: return hipErrorInvalidValue;
    }
}

namespace {

// rows [0, S) of a [b, S, W] fp32 tensor with element strides (sb, ss) set
// to zero (a strided view: elements between its rows are not touched)
__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ p, int S, int W, int64_t n, int64_t sb,
                                                        int64_t ss)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / W;
        p[(row / S) * sb + (row % S) * ss + i % W] = 0.f;
    }
}

hipError_t zero_rows(float* p, int b, int S, int W, int64_t sb, int64_t ss, hipStream_t st)
{
    const int64_t n = (int64_t)b * S * W;
    if (n == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, S, W, n, sb, ss);
    return hipGetLastError();
}

}  // namespace

hipError_t compress_bwd(const CompressArgs& p, bool bf16, hipStream_t st)
{
    if (p.nc == 0) {     // no block: every gradient row is zero, and so is the weight gradient
        hipError_t e = zero_rows(p.dx, p.b, p.S, p.D, p.xsb, p.xss, st);
        if (e == hipSuccess) e = zero_rows(p.dz, p.b, p.S, p.zc, p.zsb, p.zss, st);
        if (e == hipSuccess && p.dnorm_w) e = zero_fill(p.dnorm_w, (size_t)p.D, st);
        return e;
    }
    switch (p.D) {
    case 64: return bf16 ? compress_bwd_d<bf16_t, 64>(p, st) : compress_bwd_d<float, 64>(p, st);
    case 128: return bf16 ? compress_bwd_d<bf16_t, 128>(p, st) : compress_bwd_d<float, 128>(p, st);
    case 512: return bf16 ? compress_bwd_d<bf16_t, 512>(p, st) : compress_bwd_d<float, 512>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csa
