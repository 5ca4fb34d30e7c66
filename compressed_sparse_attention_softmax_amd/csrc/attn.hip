// attn.hip -- sparse attention forward and backward over window + selected
// compressed rows + per-head sink (gfx950).
//
// Megatron-LM PR #6400 (gather thread): each query gathers its candidate rows
// from the compact KV and the compressed rows, and the backward accumulates
// into those compact buffers instead of a [b, sq, n_kv, d] gradient.  Same
// PR, sink thread: a per-head fp32 logit joins the softmax denominator only.
// torchtitan PR #4452: window rows, selected compressed rows and the sink
// share one softmax, and the per-head LSE is returned; the backward is the
// sum of a probability x grad-output product and a scaled grad-score x query
// product.  Megatron-LM PR #7152: selected gradients are scattered back to
// positions in fp32 so repeated indices lose nothing.
//
// One KV head serves all h query heads, so the rows a query gathers are
// shared by its heads: the natural matrix-core tile is (heads x gathered
// rows x d).  A wave owns one query and a group of 16*HT heads and walks its
// candidate list in chunks of 32 rows ("slots": the window rows first, then
// the compressed slots).  Rows are loaded straight from global memory into
// MFMA operand registers (16-byte row segments); a wave-private LDS tile
// holds the same rows for the contractions over rows, whose operand needs 8
// rows at one column per lane.
#include "csa_device.hpp"
#include "csa_kernels.hpp"

namespace csa {

namespace {

constexpr int CHUNK = 32;

template <typename T> constexpr int row_pad() { return 16 / (int)sizeof(T); }

// Candidate list of one query.
template <typename T>
struct Cand {
    const T* kv;          // batch base of kv
    const T* c;           // batch base of c (nullptr: window only)
    const int32_t* irow;  // index row of the query (nullptr: dense mode)
    int t, D, u0, nwin, nv, nslots;

    __device__ __forceinline__ void init(const AttnArgs& p, int bi, int tq)
    {
        t = tq;
        D = p.D;
        kv = (const T*)p.kv + (int64_t)bi * p.S * p.D;
        c = p.c ? (const T*)p.c + (int64_t)bi * p.nc * p.D : nullptr;
        irow = (p.c && p.idx) ? p.idx + ((int64_t)bi * p.S + tq) * p.kp : nullptr;
        nwin = min(p.W, tq + 1);
        u0 = tq - nwin + 1;
        nv = p.c ? min((tq + 1) / p.r, p.nc) : 0;
        const int ncs = p.c ? (p.idx ? p.kp : nv) : 0;
        nslots = nwin + ncs;
    }
    // row of a slot: kind 0 = window row u, 1 = compressed row j, -1 = invalid
    __device__ __forceinline__ int locate(int slot, int& where) const
    {
        if (slot < nwin) { where = u0 + slot; return 0; }
        if (slot >= nslots) { where = t; return -1; }
        const int s2 = slot - nwin;
        const int j = irow ? irow[s2] : s2;
        if (j < 0 || j >= nv) { where = t; return -1; }
        where = j;
        return 1;
    }
    __device__ __forceinline__ const T* row_ptr(int kind, int where) const
    {
        return kind == 1 ? c + (int64_t)where * D : kv + (int64_t)where * D;
    }
    // bit s of the result: slot c0 + s is a valid candidate (s < 32)
    __device__ __forceinline__ uint32_t chunk_mask(int c0) const
    {
        int where;
        const bool v = locate(c0 + (lane_id() & 31), where) >= 0;
        return (uint32_t)__ballot(v);
    }
};

// ---------------------------------------------------------------- forward
// S^T[r, h] = R[r, :] . Q[h, :]        A = gathered rows (m = r, k = d),
//                                      B = Q^T (k = d, n = h), registers
// online softmax per column h (lane), base-2 exponentials
// O^T[d, h] += R^T[d, r] P^T[r, h]     A = R^T from the LDS tile (8 rows at
//                                      one column per lane), B = P^T straight
//                                      from the S^T accumulators: lane (h, g)
//                                      holds rows 4g+i of row tiles 0 and 1,
//                                      i.e. k = 8g + e <-> r = 16(e/4) + 4g + e%4
template <typename T, int D, int HT, int G>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs p)
{
    constexpr int KS = D / 32, DT = D / 16, QPW = 4 / G;
    constexpr int ROW = D + row_pad<T>();
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int g = lane / 16, n16 = lane % 16;
    T* tile = reinterpret_cast<T*>(smem) + (size_t)wave * CHUNK * ROW;

    const int bi = blockIdx.y;
    const int t = blockIdx.x * QPW + wave / G;
    if (t >= p.S) return;
    const int h0 = (wave % G) * 16 * HT;
    Cand<T> cand;
    cand.init(p, bi, t);
    const int64_t qrow = (int64_t)bi * p.S + t;
    const float sl2 = p.scale * LOG2E;

    Frag<T> qb[HT][KS];
    float m2[HT], l[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + 16 * ht + n16;
        const bool hv = h < p.H;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ht][ks] = hv ? load_frag((const T*)p.q + (qrow * p.H + h) * D + 32 * ks + 8 * g) : zero_frag<T>();
        if (p.sink && hv) { m2[ht] = p.sink[h] * LOG2E; l[ht] = 1.f; }
        else { m2[ht] = -INFINITY; l[ht] = 0.f; }
    }
    f32x4 o[DT][HT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o[dt][ht] = f4zero();

    for (int c0 = 0; c0 < cand.nslots; c0 += CHUNK) {
        const uint32_t mask = cand.chunk_mask(c0);
        if (mask == 0u) continue;
        // gathered rows as A operands (m = r), copied to the LDS tile
        Frag<T> ra[2][KS];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            int where;
            const int kind = cand.locate(c0 + 16 * rt + n16, where);
            const T* src = cand.row_ptr(kind, where);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ra[rt][ks] = load_frag(src + 32 * ks + 8 * g);
                store_frag(tile + (16 * rt + n16) * ROW + 32 * ks + 8 * g, ra[rt][ks]);
            }
        }
        f32x4 s[2][HT];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                f32x4 acc = f4zero();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma16(ra[rt][ks], qb[ht][ks], acc);
                s[rt][ht] = acc;
            }
        Frag<T> pb[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float x[2][4];
            float mx = -INFINITY;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool v = (mask >> (16 * rt + 4 * g + i)) & 1u;
                    x[rt][i] = v ? s[rt][ht][i] * sl2 : -INFINITY;
                    mx = fmaxf(mx, x[rt][i]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m2[ht], mx);
            const float alpha = exp2f(m2[ht] - mnew);
            float rs = 0.f;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = exp2f(x[rt][i] - mnew);
                    rs += pv;
                    pb[ht].v[4 * rt + i] = from_f32<T>(pv);
                }
            rs += __shfl_xor(rs, 16);
            rs += __shfl_xor(rs, 32);
            l[ht] = l[ht] * alpha + rs;
            m2[ht] = mnew;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][ht] *= alpha;
        }
        // O^T += R^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            Frag<T> a;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a.v[e] = tile[(16 * (e / 4) + 4 * g + (e % 4)) * ROW + 16 * dt + n16];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) o[dt][ht] = mfma16(a, pb[ht], o[dt][ht]);
        }
    }
    // epilogue: O[t, h, d] = O^T[d, h] / l;  lse = (m2 + log2 l) ln 2
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + 16 * ht + n16;
        if (h >= p.H) continue;
        const float inv = 1.f / l[ht];
        T* orow = (T*)p.out + (qrow * p.H + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * g + i] = from_f32<T>(o[dt][ht][i] * inv);
        }
        if (g == 0) p.lse[qrow * p.H + h] = (m2[ht] + log2f(l[ht])) * LN2;
    }
}

// --------------------------------------------------------------- backward
// S[h, r]  = Q[h, :] . R[r, :]       A = Q (m = h, k = d), B = R (k = d, n = r)
// dP[h, r] = dO[h, :] . R[r, :]      same B operand
// P = exp(scale S - lse), dS' = scale P (dP - Delta)
// dR[r, d] = P^T dO + dS'^T Q        A = P^T / dS'^T straight from the S/dP
//                                    accumulators (lane (r, g) holds heads 4g+i
//                                    of head tiles 0 and 1: k = 8g + e <->
//                                    head 16(e/4) + 4g + e%4), B = dO / Q
//                                    gathered once per query in that head order
//                                    -> fp32 atomics into dkv / dc
// dQ[h, d] += dS'[h, :] R[:, d]      A = dS' through an LDS tile [h][r],
//                                    B = R^T from the row tile
template <typename T, int D, int HT, int G>
__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(AttnArgs p)
{
    constexpr int KS = D / 32, DT = D / 16, QPW = 4 / G;
    constexpr int ROW = D + row_pad<T>();
    constexpr int DSROW = CHUNK + row_pad<T>();
    static_assert(HT <= 2, "one k-step of 32 heads per dR product");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int g = lane / 16, n16 = lane % 16;
    const size_t wave_elems = (size_t)CHUNK * ROW + (size_t)16 * HT * DSROW;
    T* tile = reinterpret_cast<T*>(smem) + (size_t)wave * wave_elems;
    T* dstile = tile + (size_t)CHUNK * ROW;

    const int bi = blockIdx.y;
    const int t = blockIdx.x * QPW + wave / G;
    if (t >= p.S) return;
    const int h0 = (wave % G) * 16 * HT;
    Cand<T> cand;
    cand.init(p, bi, t);
    const int64_t qrow = (int64_t)bi * p.S + t;
    const T* qp = (const T*)p.q + qrow * p.H * D;
    const T* dop = (const T*)p.dout + qrow * p.H * D;
    const T* op = (const T*)p.out + qrow * p.H * D;
    const float sl2 = p.scale * LOG2E;

    // Delta[h] = <dO[t, h], O[t, h]> for the wave's heads, kept in C-row layout
    float lse2[HT][4], dlt[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = h0 + 16 * ht + 4 * g + i;
            lse2[ht][i] = h < p.H ? p.lse[qrow * p.H + h] * LOG2E : 0.f;
            dlt[ht][i] = 0.f;
        }
    for (int hh = 0; hh < 16 * HT; ++hh) {
        const int h = h0 + hh;
        if (h >= p.H) break;
        float part = 0.f;
        for (int d = lane; d < D; d += WAVE) part += to_f32(dop[h * D + d]) * to_f32(op[h * D + d]);
        part = wave_sum(part);
        const int ht = hh / 16, gg = (hh % 16) / 4, ii = hh % 4;
#pragma unroll
        for (int a = 0; a < HT; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (a == ht && g == gg && i == ii) dlt[a][i] = part;
    }
    if (p.dsink && p.sink && n16 == 0) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = h0 + 16 * ht + 4 * g + i;
                if (h < p.H) atomicAdd(p.dsink + h, -exp2f(p.sink[h] * LOG2E - lse2[ht][i]) * dlt[ht][i]);
            }
    }
    if (!p.dq) return;

    Frag<T> qa[HT][KS], da[HT][KS];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + 16 * ht + n16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bool hv = h < p.H;
            qa[ht][ks] = hv ? load_frag(qp + h * D + 32 * ks + 8 * g) : zero_frag<T>();
            da[ht][ks] = hv ? load_frag(dop + h * D + 32 * ks + 8 * g) : zero_frag<T>();
        }
    }
    // B operands of dR (k = head in the order 16(e/4) + 4g + e%4, n = d)
    Frag<T> dob[DT], qbb[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int hk = 16 * (e / 4) + 4 * g + (e % 4);
            const int h = h0 + hk;
            const bool hv = hk < 16 * HT && h < p.H;
            dob[dt].v[e] = hv ? dop[h * D + 16 * dt + n16] : from_f32<T>(0.f);
            qbb[dt].v[e] = hv ? qp[h * D + 16 * dt + n16] : from_f32<T>(0.f);
        }
    f32x4 dq[HT][DT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dq[ht][dt] = f4zero();

    float* dkv_b = p.dkv + (int64_t)bi * p.S * D;
    float* dc_b = p.dc ? p.dc + (int64_t)bi * p.nc * D : nullptr;

    for (int c0 = 0; c0 < cand.nslots; c0 += CHUNK) {
        const uint32_t mask = cand.chunk_mask(c0);
        if (mask == 0u) continue;
        Frag<T> rb[2][KS];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            int where;
            const int kind = cand.locate(c0 + 16 * rt + n16, where);
            const T* src = cand.row_ptr(kind, where);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                rb[rt][ks] = load_frag(src + 32 * ks + 8 * g);
                store_frag(tile + (16 * rt + n16) * ROW + 32 * ks + 8 * g, rb[rt][ks]);
            }
        }
        Frag<T> pa[2], sa[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            pa[rt] = zero_frag<T>();
            sa[rt] = zero_frag<T>();
            const bool rv = (mask >> (16 * rt + n16)) & 1u;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                f32x4 sacc = f4zero(), pacc = f4zero();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    sacc = mfma16(qa[ht][ks], rb[rt][ks], sacc);
                    pacc = mfma16(da[ht][ks], rb[rt][ks], pacc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = rv ? exp2f(sacc[i] * sl2 - lse2[ht][i]) : 0.f;
                    const float dsv = p.scale * pv * (pacc[i] - dlt[ht][i]);
                    pa[rt].v[4 * ht + i] = from_f32<T>(pv);
                    sa[rt].v[4 * ht + i] = from_f32<T>(dsv);
                    // dS' tile [h][r] for the dQ product
                    dstile[(16 * ht + 4 * g + i) * DSROW + 16 * rt + n16] = from_f32<T>(dsv);
                }
            }
        }
        // dR = P^T dO + dS'^T Q, scattered with fp32 atomics
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float* dst[4];
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int where;
                const int kind = cand.locate(c0 + 16 * rt + 4 * g + i, where);
                ok[i] = kind >= 0;
                dst[i] = kind == 1 ? dc_b + (int64_t)where * D : dkv_b + (int64_t)where * D;
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                f32x4 acc = mfma16(pa[rt], dob[dt], f4zero());
                acc = mfma16(sa[rt], qbb[dt], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (ok[i]) atomicAdd(dst[i] + 16 * dt + n16, acc[i]);
            }
        }
        // dQ += dS' R
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const Frag<T> a = load_frag(dstile + (16 * ht + n16) * DSROW + 8 * g);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                Frag<T> bfr;
#pragma unroll
                for (int e = 0; e < 8; ++e) bfr.v[e] = tile[(8 * g + e) * ROW + 16 * dt + n16];
                dq[ht][dt] = mfma16(a, bfr, dq[ht][dt]);
            }
        }
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = h0 + 16 * ht + 4 * g + i;
            if (h >= p.H) continue;
            T* dqrow = (T*)p.dq + (qrow * p.H + h) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) dqrow[16 * dt + n16] = from_f32<T>(dq[ht][dt][i]);
        }
}

template <typename T, int D, int HT>
hipError_t launch_fwd(const AttnArgs& p, hipStream_t st)
{
    const int gper = (p.H + 16 * HT - 1) / (16 * HT);
    const size_t lds = (size_t)4 * CHUNK * (D + row_pad<T>()) * sizeof(T);
    if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    auto go = [&](auto kern, int qpw) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        dim3 grid((p.S + qpw - 1) / qpw, p.b);
        hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, p);
        return hipGetLastError();
    };
    switch (gper) {
    case 1: return go(attn_fwd_kernel<T, D, HT, 1>, 4);
    case 2: return go(attn_fwd_kernel<T, D, HT, 2>, 2);
    case 3:
    case 4: return go(attn_fwd_kernel<T, D, HT, 4>, 1);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D, int HT>
hipError_t launch_bwd(const AttnArgs& p, hipStream_t st)
{
    const int gper = (p.H + 16 * HT - 1) / (16 * HT);
    const size_t lds = (size_t)4 * (CHUNK * (D + row_pad<T>()) + 16 * HT * (CHUNK + row_pad<T>())) * sizeof(T);
    if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    auto go = [&](auto kern, int qpw) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        dim3 grid((p.S + qpw - 1) / qpw, p.b);
        hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, p);
        return hipGetLastError();
    };
    switch (gper) {
    case 1: return go(attn_bwd_kernel<T, D, HT, 1>, 4);
    case 2: return go(attn_bwd_kernel<T, D, HT, 2>, 2);
    case 3:
    case 4: return go(attn_bwd_kernel<T, D, HT, 4>, 1);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t fwd_dispatch(const AttnArgs& p, hipStream_t st)
{
    switch (p.D) {
    case 64: return p.H <= 16 ? launch_fwd<T, 64, 1>(p, st) : p.H <= 32 ? launch_fwd<T, 64, 2>(p, st) : launch_fwd<T, 64, 4>(p, st);
    case 128: return p.H <= 16 ? launch_fwd<T, 128, 1>(p, st) : p.H <= 32 ? launch_fwd<T, 128, 2>(p, st) : launch_fwd<T, 128, 4>(p, st);
    case 512: return launch_fwd<T, 512, 1>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t bwd_dispatch(const AttnArgs& p, hipStream_t st)
{
    switch (p.D) {
    case 64: return p.H <= 16 ? launch_bwd<T, 64, 1>(p, st) : launch_bwd<T, 64, 2>(p, st);
    case 128: return p.H <= 16 ? launch_bwd<T, 128, 1>(p, st) : launch_bwd<T, 128, 2>(p, st);
    case 512: return launch_bwd<T, 512, 1>(p, st);
    default: return hipErrorInvalidValue;
    }
}

__global__ void zero_fill_kernel(float* __restrict__ p, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) *reinterpret_cast<float4*>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
        else for (size_t k = i; k < n; ++k) p[k] = 0.f;
    }
}

}  // namespace

hipError_t attn_fwd(const AttnArgs& p, bool bf16, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    return bf16 ? fwd_dispatch<bf16_t>(p, st) : fwd_dispatch<float>(p, st);
}

hipError_t attn_bwd(const AttnArgs& p, bool bf16, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    return bf16 ? bwd_dispatch<bf16_t>(p, st) : bwd_dispatch<float>(p, st);
}

hipError_t zero_fill(float* p, size_t n, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    size_t blocks = (n / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace csa
