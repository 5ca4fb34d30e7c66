// dsa_gqa.hip -- simplified DSA over grouped-query attention (gfx950).
//
// Megatron-LM PR #7152: a one-head indexer without per-head weights selects
// K' keys per query at full resolution (csa_index_topk with ratio 1, one
// head and unit weights), and attention runs over the selected keys only,
// query head h reading key/value head g = h / (H / H_kv), keys and values
// being separate tensors.
//
// The attention kernels of attn.hip take one row per key that serves as both
// key and value.  Keys and values of group g are therefore packed into one
// row [k | v] of width d_qk + d_v, queries into [q | 0] and, in the
// backward, dO into [0 | dO] and O into [0 | O]; with no window (W = 0), no
// sink and ratio 1 the packed rows act as the "compressed" rows selected by
// the index list (the kernels, told where the key half ends, skip the
// products with a zero half at d_qk + d_v = 256), and
//   logits  = <[q | 0], [k | v]>            = <q, k>
//   O'      = sum P [k | v],                  O = its v half
//   Delta   = <[0 | dO], [0 | O]>           = <dO, O>
//   dq'     = scale sum dS [k | v],           dq = its k half
//   drow    = sum P [0 | dO] + scale dS [q | 0] = [dk | dv].
// The groups run one after another on the caller's stream; the packing and
// unpacking kernels are plain element-wise copies.  At other widths the zero
// halves cost matrix-core work (about half of each product).
#include "csa_device.hpp"
#include "csa_kernels.hpp"

namespace csa {

namespace {

constexpr int NT = 256;

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

struct Layout {
    size_t rows, q, out, lse, dout, dq, dc, dkv, attn, sel, total;
    int selw;   // words per selection-bitmap row (0: no bitmap)
};

AttnArgs group_args(const GqaArgs& p)
{
    AttnArgs a{};
    a.scale = p.scale;
    a.idx = p.idx;
    a.b = p.b; a.S = p.S; a.H = p.H / p.HKV; a.D = p.DK + p.DV; a.W = 0; a.r = 1; a.nc = p.S; a.kp = p.kp;
    // the kernels skip the zero halves when the key half is whole k-steps
    a.dsplit = (p.DK % 32 == 0) ? p.DK : 0;
    return a;
}

Layout layout(const GqaArgs& p, size_t e, bool bwd)
{
    const size_t Dp = p.DK + p.DV, hg = p.H / p.HKV, bs = (size_t)p.b * p.S;
    Layout l{};
    size_t off = 0;
    l.rows = off; off += align256((size_t)p.HKV * bs * Dp * e);
    l.q = off;    off += align256(bs * hg * Dp * e);
    l.out = off;  off += align256(bs * hg * Dp * e);
    l.lse = off;  off += align256(bs * hg * 4);
    if (bwd) {
        AttnArgs a = group_args(p);
        a.c = a.kv = a.q = reinterpret_cast<const void*>(16);
        l.dout = off; off += align256(bs * hg * Dp * e);
        l.dq = off;   off += align256(bs * hg * Dp * e);
        l.dc = off;   off += align256(bs * Dp * 4);
        l.dkv = off;  off += align256(bs * Dp * 4);
        l.attn = off; off += align256(attn_bwd_workspace_bytes(a));
        // the selection bitmap, built once and read by every group's backward
        a.idx = reinterpret_cast<const int32_t*>(16);
        l.selw = attn_bwd_stacks_queries(a, e == 2) ? selmap_words(a) : 0;
        l.sel = off;  off += align256((size_t)p.b * p.S * l.selw * 4);
    }
    l.total = off;
    return l;
}

// rows[g, b, s, :] = [k[b, s, g, :] | v[b, s, g, :]]
template <typename T>
__global__ __launch_bounds__(NT) void pack_rows_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                       T* __restrict__ rows, int64_t bs, int hkv, int dk, int dv)
{
    const int dp = dk + dv;
    const int64_t n = (int64_t)hkv * bs * dp;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int c = (int)(i % dp);
        const int64_t gs = i / dp;
        const int64_t s = gs % bs;
        const int g = (int)(gs / bs);
        rows[i] = c < dk ? k[(s * hkv + g) * dk + c] : v[(s * hkv + g) * dv + (c - dk)];
    }
}

// dst[b, s, hl, :] = [zeros(lo) | src[b, s, g * hg + hl, :] | zeros(hi)] with
// the source row placed at column `at` (0: the k half, dk: the v half)
template <typename T>
__global__ __launch_bounds__(NT) void pack_heads_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t bs,
                                                        int H, int hg, int g, int w, int dp, int at)
{
    const int64_t n = bs * hg * dp;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int c = (int)(i % dp);
        const int64_t sh = i / dp;
        const int hl = (int)(sh % hg);
        const int64_t s = sh / hg;
        const int cc = c - at;
        dst[i] = (cc >= 0 && cc < w) ? src[(s * H + g * hg + hl) * w + cc] : (T)0.0f;
    }
}

// dst[b, s, g * hg + hl, :] = src[b, s, hl, at : at + w]  (dst of type U)
template <typename T, typename U>
__global__ __launch_bounds__(NT) void unpack_heads_kernel(const T* __restrict__ src, U* __restrict__ dst, int64_t bs,
                                                          int H, int hg, int g, int w, int dp, int at)
{
    const int64_t n = bs * hg * w;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int c = (int)(i % w);
        const int64_t sh = i / w;
        const int hl = (int)(sh % hg);
        const int64_t s = sh / hg;
        dst[(s * H + g * hg + hl) * w + c] = (U)to_f32(src[(s * hg + hl) * dp + at + c]);
    }
}

// lse[b, s, g * hg + hl] = src[b, s, hl], or the reverse (to_group)
__global__ __launch_bounds__(NT) void move_lse_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                      int64_t bs, int H, int hg, int g, int to_group)
{
    const int64_t n = bs * hg;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int64_t s = i / hg;
        const int hl = (int)(i % hg);
        const int64_t full = s * H + g * hg + hl;
        if (to_group) dst[i] = src[full];
        else dst[full] = src[i];
    }
}

// dk[b, s, g, :] = dc[b, s, 0:dk], dv[b, s, g, :] = dc[b, s, dk:]
__global__ __launch_bounds__(NT) void unpack_kv_kernel(const float* __restrict__ dc, float* __restrict__ dkk,
                                                       float* __restrict__ dvv, int64_t bs, int hkv, int g, int dk,
                                                       int dv)
{
    const int dp = dk + dv;
    const int64_t n = bs * dp;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int c = (int)(i % dp);
        const int64_t s = i / dp;
        if (c < dk) dkk[(s * hkv + g) * dk + c] = dc[i];
        else dvv[(s * hkv + g) * dv + (c - dk)] = dc[i];
    }
}

dim3 grid_for(int64_t n)
{
    int64_t blocks = (n + NT - 1) / NT;
    return dim3((unsigned)(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192));
}

template <typename T>
hipError_t run_fwd(const GqaArgs& p, char* ws, hipStream_t st)
{
    const Layout l = layout(p, sizeof(T), false);
    const int hg = p.H / p.HKV, dp = p.DK + p.DV;
    const int64_t bs = (int64_t)p.b * p.S;
    T* rows = reinterpret_cast<T*>(ws + l.rows);
    T* qg = reinterpret_cast<T*>(ws + l.q);
    T* og = reinterpret_cast<T*>(ws + l.out);
    float* lg = reinterpret_cast<float*>(ws + l.lse);
    hipLaunchKernelGGL(pack_rows_kernel<T>, grid_for((int64_t)p.HKV * bs * dp), dim3(NT), 0, st, (const T*)p.k,
                       (const T*)p.v, rows, bs, p.HKV, p.DK, p.DV);
    hipError_t e = hipGetLastError();
    for (int g = 0; g < p.HKV && e == hipSuccess; ++g) {
        hipLaunchKernelGGL(pack_heads_kernel<T>, grid_for(bs * hg * dp), dim3(NT), 0, st, (const T*)p.q, qg, bs,
                           p.H, hg, g, p.DK, dp, 0);
        if ((e = hipGetLastError()) != hipSuccess) break;
        AttnArgs a = group_args(p);
        a.q = qg;
        a.kv = a.c = rows + (size_t)g * bs * dp;
        a.out = og;
        a.lse = lg;
        if ((e = attn_fwd(a, sizeof(T) == 2, st)) != hipSuccess) break;
        hipLaunchKernelGGL((unpack_heads_kernel<T, T>), grid_for(bs * hg * p.DV), dim3(NT), 0, st, og, (T*)p.out, bs,
                           p.H, hg, g, p.DV, dp, p.DK);
        hipLaunchKernelGGL(move_lse_kernel, grid_for(bs * hg), dim3(NT), 0, st, lg, p.lse, bs, p.H, hg, g, 0);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
hipError_t run_bwd(const GqaArgs& p, char* ws, hipStream_t st)
{
    const Layout l = layout(p, sizeof(T), true);
    const int hg = p.H / p.HKV, dp = p.DK + p.DV;
    const int64_t bs = (int64_t)p.b * p.S;
    T* rows = reinterpret_cast<T*>(ws + l.rows);
    T* qg = reinterpret_cast<T*>(ws + l.q);
    T* og = reinterpret_cast<T*>(ws + l.out);
    float* lg = reinterpret_cast<float*>(ws + l.lse);
    T* dog = reinterpret_cast<T*>(ws + l.dout);
    T* dqg = reinterpret_cast<T*>(ws + l.dq);
    float* dcg = reinterpret_cast<float*>(ws + l.dc);
    float* dkvg = reinterpret_cast<float*>(ws + l.dkv);
    float* aws = reinterpret_cast<float*>(ws + l.attn);
    uint32_t* sel = l.selw ? reinterpret_cast<uint32_t*>(ws + l.sel) : nullptr;
    hipLaunchKernelGGL(pack_rows_kernel<T>, grid_for((int64_t)p.HKV * bs * dp), dim3(NT), 0, st, (const T*)p.k,
                       (const T*)p.v, rows, bs, p.HKV, p.DK, p.DV);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sel) e = build_selmap(group_args(p), sel, st);
    for (int g = 0; g < p.HKV && e == hipSuccess; ++g) {
        hipLaunchKernelGGL(pack_heads_kernel<T>, grid_for(bs * hg * dp), dim3(NT), 0, st, (const T*)p.q, qg, bs,
                           p.H, hg, g, p.DK, dp, 0);
        hipLaunchKernelGGL(pack_heads_kernel<T>, grid_for(bs * hg * dp), dim3(NT), 0, st, (const T*)p.out, og, bs,
                           p.H, hg, g, p.DV, dp, p.DK);
        hipLaunchKernelGGL(pack_heads_kernel<T>, grid_for(bs * hg * dp), dim3(NT), 0, st, (const T*)p.dout, dog, bs,
                           p.H, hg, g, p.DV, dp, p.DK);
        hipLaunchKernelGGL(move_lse_kernel, grid_for(bs * hg), dim3(NT), 0, st, p.lse, lg, bs, p.H, hg, g, 1);
        if ((e = hipGetLastError()) != hipSuccess) break;
        AttnArgs a = group_args(p);
        a.q = qg;
        a.kv = a.c = rows + (size_t)g * bs * dp;
        a.out = og;
        a.lse = lg;
        a.dout = dog;
        a.dq = dqg;
        a.dkv = dkvg;
        a.dc = dcg;
        a.selmap = sel;
        a.selw = l.selw;
        if ((e = attn_bwd(a, sizeof(T) == 2, aws, st)) != hipSuccess) break;
        hipLaunchKernelGGL((unpack_heads_kernel<T, T>), grid_for(bs * hg * p.DK), dim3(NT), 0, st, dqg, (T*)p.dq, bs,
                           p.H, hg, g, p.DK, dp, 0);
        hipLaunchKernelGGL(unpack_kv_kernel, grid_for(bs * dp), dim3(NT), 0, st, dcg, p.dk, p.dv, bs, p.HKV, g, p.DK,
                           p.DV);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

size_t dsa_gqa_workspace_bytes(const GqaArgs& p, bool bf16, bool bwd)
{
    return layout(p, bf16 ? 2 : 4, bwd).total;
}

hipError_t dsa_gqa_fwd(const GqaArgs& p, bool bf16, void* ws, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    return bf16 ? run_fwd<bf16_t>(p, (char*)ws, st) : run_fwd<float>(p, (char*)ws, st);
}

hipError_t dsa_gqa_bwd(const GqaArgs& p, bool bf16, void* ws, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    return bf16 ? run_bwd<bf16_t>(p, (char*)ws, st) : run_bwd<float>(p, (char*)ws, st);
}

}  // namespace csa
