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
#include <initializer_list>

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
    a.set_contiguous();                       // the packed buffers are batch-major
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

// The copies below move whole 16-byte units (U = uint4) when every width is
// a multiple of one and every tensor is 16-byte aligned, else single
// elements (U = the element type); widths and offsets are in units of U.

// rows[g, b, s, :] = [k[b, s, g, :] | v[b, s, g, :]]
template <typename U>
__global__ __launch_bounds__(NT) void pack_rows_kernel(const U* __restrict__ k, const U* __restrict__ v,
                                                       U* __restrict__ rows, int64_t bs, int hkv, int dk, int dv)
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

// Heads g*hg + hl of q (and, in the backward, of O and dO) into the group's
// packed buffers [q | 0], [0 | O], [0 | dO].  The zero halves are written
// only when `zeros` (the buffers are reused group after group and the halves
// stay zero); the backward also gathers the group's LSE columns.
template <typename U>
__global__ __launch_bounds__(NT) void pack_group_kernel(const U* __restrict__ q, const U* __restrict__ out,
                                                        const U* __restrict__ dout, U* __restrict__ qg,
                                                        U* __restrict__ og, U* __restrict__ dog,
                                                        const float* __restrict__ lse, float* __restrict__ lg,
                                                        int64_t bs, int H, int hg, int g, int dk, int dv, int zeros)
{
    const int dp = dk + dv;
    const int64_t n = bs * hg * dp;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int c = (int)(i % dp);
        const int64_t sh = i / dp;                                  // s * hg + hl
        const int64_t srow = (sh / hg) * H + g * hg + sh % hg;      // row of the full-head tensors
        if (c < dk) {
            qg[i] = q[srow * dk + c];
            if (zeros && og) {
                og[i] = U{};
                dog[i] = U{};
            }
        } else {
            if (og) {
                og[i] = out[srow * dv + (c - dk)];
                dog[i] = dout[srow * dv + (c - dk)];
            }
            if (zeros) qg[i] = U{};
        }
        if (lg && c == 0) lg[sh] = lse[srow];
    }
}

// dst[b, s, g * hg + hl, :] = src[b, s, hl, at : at + w], and (forward) the
// group's LSE columns back into the full-head LSE
template <typename U>
__global__ __launch_bounds__(NT) void unpack_group_kernel(const U* __restrict__ src, U* __restrict__ dst,
                                                          const float* __restrict__ lg, float* __restrict__ lse,
                                                          int64_t bs, int H, int hg, int g, int w, int dp, int at)
{
    const int64_t n = bs * hg * w;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
        const int c = (int)(i % w);
        const int64_t sh = i / w;
        const int64_t srow = (sh / hg) * H + g * hg + sh % hg;
        dst[srow * w + c] = src[sh * dp + at + c];
        if (lse && c == 0) lse[srow] = lg[sh];
    }
}

// dk[b, s, g, :] = dc[b, s, 0:dk], dv[b, s, g, :] = dc[b, s, dk:]   (fp32)
template <typename U>
__global__ __launch_bounds__(NT) void unpack_kv_kernel(const U* __restrict__ dc, U* __restrict__ dkk,
                                                       U* __restrict__ dvv, int64_t bs, int hkv, int g, int dk, int dv)
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

bool units16(std::initializer_list<const void*> ptrs, std::initializer_list<int64_t> bytes)
{
    for (const void* q : ptrs)
        if (((uintptr_t)q) & 15) return false;
    for (int64_t b : bytes)
        if (b % 16) return false;
    return true;
}

// element copies in units of U: V elements of T per unit
template <typename T, typename U>
struct Packer {
    static constexpr int V = (int)(sizeof(U) / sizeof(T));
    const GqaArgs& p;
    int64_t bs;
    int hg, dp;
    hipStream_t st;

    void rows(T* dst) const
    {
        const int64_t n = (int64_t)p.HKV * bs * dp / V;
        hipLaunchKernelGGL(pack_rows_kernel<U>, grid_for(n), dim3(NT), 0, st, (const U*)p.k, (const U*)p.v, (U*)dst, bs,
                           p.HKV, p.DK / V, p.DV / V);
    }
    void group_in(int g, T* qg, T* og, T* dog, float* lg, bool zeros) const
    {
        hipLaunchKernelGGL(pack_group_kernel<U>, grid_for(bs * hg * dp / V), dim3(NT), 0, st, (const U*)p.q,
                           (const U*)p.out, (const U*)p.dout, (U*)qg, (U*)og, (U*)dog, p.lse, lg, bs, p.H, hg, g,
                           p.DK / V, p.DV / V, zeros ? 1 : 0);
    }
    void group_out(int g, const T* src, T* dst, const float* lg, float* lse, int w, int at) const
    {
        hipLaunchKernelGGL(unpack_group_kernel<U>, grid_for(bs * hg * w / V), dim3(NT), 0, st, (const U*)src, (U*)dst,
                           lg, lse, bs, p.H, hg, g, w / V, dp / V, at / V);
    }
};

template <typename U>
void unpack_kv(const GqaArgs& p, const float* dc, int64_t bs, int g, hipStream_t st)
{
    constexpr int V = (int)(sizeof(U) / sizeof(float));
    hipLaunchKernelGGL(unpack_kv_kernel<U>, grid_for(bs * (p.DK + p.DV) / V), dim3(NT), 0, st, (const U*)dc, (U*)p.dk,
                       (U*)p.dv, bs, p.HKV, g, p.DK / V, p.DV / V);
}

template <typename T, typename U>
hipError_t run_fwd_u(const GqaArgs& p, char* ws, hipStream_t st)
{
    const Layout l = layout(p, sizeof(T), false);
    const int hg = p.H / p.HKV, dp = p.DK + p.DV;
    const int64_t bs = (int64_t)p.b * p.S;
    T* rows = reinterpret_cast<T*>(ws + l.rows);
    T* qg = reinterpret_cast<T*>(ws + l.q);
    T* og = reinterpret_cast<T*>(ws + l.out);
    float* lg = reinterpret_cast<float*>(ws + l.lse);
    const Packer<T, U> pk{p, bs, hg, dp, st};
    pk.rows(rows);
    hipError_t e = hipGetLastError();
    for (int g = 0; g < p.HKV && e == hipSuccess; ++g) {
        pk.group_in(g, qg, nullptr, nullptr, nullptr, g == 0);
        if ((e = hipGetLastError()) != hipSuccess) break;
        AttnArgs a = group_args(p);
        a.q = qg;
        a.kv = a.c = rows + (size_t)g * bs * dp;
        a.out = og;
        a.lse = lg;
        if ((e = attn_fwd(a, sizeof(T) == 2, st)) != hipSuccess) break;
        pk.group_out(g, og, (T*)p.out, lg, p.lse, p.DV, p.DK);
        e = hipGetLastError();
    }
    return e;
}

template <typename T, typename U, typename UF>
hipError_t run_bwd_u(const GqaArgs& p, char* ws, hipStream_t st)
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
    const Packer<T, U> pk{p, bs, hg, dp, st};
    pk.rows(rows);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sel) e = build_selmap(group_args(p), sel, st);
    for (int g = 0; g < p.HKV && e == hipSuccess; ++g) {
        pk.group_in(g, qg, og, dog, lg, g == 0);
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
        pk.group_out(g, dqg, (T*)p.dq, nullptr, nullptr, p.DK, 0);
        unpack_kv<UF>(p, dcg, bs, g, st);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
hipError_t run_fwd(const GqaArgs& p, char* ws, hipStream_t st)
{
    const int64_t e = sizeof(T);
    if (units16({p.q, p.k, p.v, p.out}, {p.DK * e, p.DV * e})) return run_fwd_u<T, uint4>(p, ws, st);
    return run_fwd_u<T, T>(p, ws, st);
}

template <typename T>
hipError_t run_bwd(const GqaArgs& p, char* ws, hipStream_t st)
{
    const int64_t e = sizeof(T);
    const bool vt = units16({p.q, p.k, p.v, p.out, p.dout, p.dq}, {p.DK * e, p.DV * e});
    const bool vf = units16({p.dk, p.dv}, {p.DK * 4, p.DV * 4});
    if (vt) return vf ? run_bwd_u<T, uint4, uint4>(p, ws, st) : run_bwd_u<T, uint4, float>(p, ws, st);
    return vf ? run_bwd_u<T, T, uint4>(p, ws, st) : run_bwd_u<T, T, float>(p, ws, st);
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
