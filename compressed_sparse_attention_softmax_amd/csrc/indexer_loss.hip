// indexer_loss.hip -- the indexer's training path (gfx950): the distillation
// loss over each query's selected blocks and its gradients into the indexer's
// inputs q_i, w and k_i.
//
// torchtitan PR #4452 (lightning indexer, indexer distillation): the teacher
// of query t is, per selected block j, the sum over attention heads of
// exp(scale <q[t,h], c[j]> - LSE[t,h]) with the attention forward's LSE
// (window, selected blocks and sink in the denominator), L1-normalised over
// the selected blocks; the student is the softmax of the indexer scores of
// the same blocks, recomputed in a second pass over the selected entries
// only.  Megatron-LM PR #6400 (teacher normalisation thread): the loss is
// KL(target || student) and its gradient with respect to the scores is
// student * sum(target) - target, zero on a zero-mass row; the per-head mass
// stays in log space so nothing underflows.  Megatron-LM PR #7152: the
// routing scores of the selected keys are reused as the student's logits,
// and gradients scattered to keys selected by many queries accumulate in
// fp32.
//
// loss_query_kernel (one workgroup per query, heads split over its 4 waves):
//   pass 1 walks the selected blocks in chunks of 32 (rows gathered into a
//   double-buffered LDS tile), forms each wave's 16 heads' logits with MFMA
//   and reduces them per block to a log2 mass; the waves' masses are
//   combined, the target, student, KL and dI = dkl (p - target) follow from
//   two block reductions; pass 2 walks the k_i rows of the same blocks,
//   recomputes a = <q_i, k_i> and accumulates dq_i^T += K^T (dI w [a > 0])^T
//   and dw += dI ReLU(a).  dI goes to the workspace.
// loss_keys_kernel (key-stationary): a workgroup owns 128 k_i rows (32 per
//   wave, kept in registers) and a block of consecutive queries; per query
//   it stages q_i and w in LDS, recomputes a for its rows, and accumulates
//   dk_i^T += q_i^T (dI w [a > 0]) over the query block, masking blocks the
//   query did not select (dI = 0).  Per-block partial rows go to the
//   workspace; loss_reduce_kernel adds them in a fixed order.
#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "timing.hpp"

namespace csa {

namespace {

constexpr int LCH = 32;        // slots per chunk in the query kernel
constexpr int NT = 256;        // threads per workgroup
constexpr int KRW = 32;        // k_i rows per wave in the keys kernel
constexpr int KTR = 4 * KRW;   // k_i rows per workgroup

// Block-wide max / sum of one float per thread (every thread gets the result).
// `red` holds 4 floats of LDS; the call contains two barriers.
__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    const int wave = threadIdx.x / WAVE;
    __syncthreads();
    if (lane_id() == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float* red)
{
    v = wave_sum(v);
    const int wave = threadIdx.x / WAVE;
    __syncthreads();
    if (lane_id() == 0) red[wave] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Gather of the 32 rows (W elements each) named by 32 consecutive slots of an
// LDS index list into registers, and their store into an LDS tile with
// 8-element units permuted per row (unit u of row r at u ^ unit_swz(r)).
// Thread i carries 16-byte pieces i, i + 256, ... of the chunk.
typedef uint32_t piece_t __attribute__((ext_vector_type(4)));   // one 16-byte piece

template <typename T, int W> constexpr int chunk_ppr() { return W * (int)sizeof(T) / 16; }
template <typename T, int W> constexpr int chunk_np() { return (LCH * chunk_ppr<T, W>() + NT - 1) / NT; }

template <typename T, int W>
__device__ __forceinline__ void chunk_fetch(piece_t* r, const T* base, const int32_t* ids, int c0)
{
    constexpr int PPR = chunk_ppr<T, W>(), NP = chunk_np<T, W>(), E16 = 16 / (int)sizeof(T);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int pc = (int)threadIdx.x + NT * k;
        const int rr = min(pc / PPR, LCH - 1), pp = pc % PPR;
        const int j = ((const lds_i32*)ids)[c0 + rr];
        r[k] = *reinterpret_cast<const piece_t*>(base + (int64_t)(j < 0 ? 0 : j) * W + pp * E16);
    }
}
template <typename T, int W>
__device__ __forceinline__ void chunk_stash(const piece_t* r, T* tile)
{
    constexpr int PPR = chunk_ppr<T, W>(), NP = chunk_np<T, W>(), E16 = 16 / (int)sizeof(T);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int pc = (int)threadIdx.x + NT * k;
        if (LCH * PPR % NT == 0 || pc < LCH * PPR) {
            const int rr = pc / PPR, pos = (pc % PPR) * E16;
            *reinterpret_cast<piece_t*>(tile + rr * W + ((((pos >> 3) ^ unit_swz(rr, W / 8))) << 3) + (pos & 7)) = r[k];
        }
    }
}

// B/A operand fragment of row r of a swizzled LDS tile (k = 32 ks + 8 g + e)
template <typename T, int W>
__device__ __forceinline__ Frag<T> tile_frag(const T* tile, int r, int ks, int g)
{
    return load_frag(tile + r * W + (((4 * ks + g) ^ unit_swz(r, W / 8)) << 3));
}

template <typename T, int D, int DI>
__global__ __launch_bounds__(NT) void loss_query_kernel(LossArgs p, float* __restrict__ gws)
{
    constexpr int KS = D / 32, KSI = DI / 32, DTI = DI / 16;
    constexpr int RW = D > DI ? D : DI;                        // elements per LDS row
    constexpr int CHB = LCH * RW * (int)sizeof(T);             // bytes per chunk tile
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x / WAVE, lane = lane_id(), g = lane / 16, n16 = lane % 16;
    const int bi = blockIdx.y;
    const int t = p.S - 1 - (int)blockIdx.x;                   // latest queries (most blocks) first
    const int64_t row = (int64_t)bi * p.S + t;
    const int kpr = (p.kp + LCH - 1) / LCH * LCH;
    T* tiles = reinterpret_cast<T*>(smem);
    float* part = reinterpret_cast<float*>(smem + 2 * CHB);    // [4][kpr] per-wave log2 masses, then a2 / dI
    int32_t* ids = reinterpret_cast<int32_t*>(part + 4 * kpr); // [kpr] block of each slot, -1 if not valid
    float* red = reinterpret_cast<float*>(ids + kpr);          // [4]
    const int nv = min((t + 1) / p.r, p.nc);
    const bool grads = p.dqi != nullptr;

    int lastv = -1;
    for (int s = threadIdx.x; s < kpr; s += NT) {
        int j = s < p.kp ? p.idx[row * p.kp + s] : -1;
        if (j < 0 || j >= nv) j = -1;
        ids[s] = j;
        if (j >= 0) lastv = s;
    }
    lastv = (int)block_max((float)lastv, red);                 // exact for slots < 2^24
    const int nch = (lastv + LCH) / LCH;

    // ---------------------------------------------------------- pass 1: teacher
    const T* qrow = (const T*)p.q + row * p.H * D;
    Frag<T> qf[KS];
    {
        const int h = 16 * wave + n16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = h < p.H ? load_frag(qrow + h * D + 32 * ks + 8 * g) : zero_frag<T>();
    }
    float lse2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 16 * wave + 4 * g + i;
        lse2[i] = h < p.H ? p.lse[row * p.H + h] * LOG2E : INFINITY;   // +inf: padded heads add nothing
    }
    const float sl2 = p.scale * LOG2E;
    const T* cb = (const T*)p.c + (int64_t)bi * p.nc * D;
    piece_t cr[chunk_np<T, D>()];
    if (nch > 0) { chunk_fetch<T, D>(cr, cb, ids, 0); chunk_stash<T, D>(cr, tiles); }
    if (nch > 1) chunk_fetch<T, D>(cr, cb, ids, LCH);
    __syncthreads();
    for (int k = 0; k < nch; ++k) {
        const T* tile = tiles + (size_t)(k & 1) * LCH * RW;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            // S[h, r] for the wave's 16 heads (m) and 16 rows (n)
            f32x4 acc = f4zero();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma16(qf[ks], tile_frag<T, D>(tile, 16 * rt + n16, ks, g), acc);
            float x[4];
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = fmaf(acc[i], sl2, -lse2[i]);
                m = fmaxf(m, x[i]);
            }
            m = rows_max(m);                                   // over the wave's 16 heads
            float sum = 0.f;
            if (m > -INFINITY) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sum += fast_exp2(x[i] - m);
            }
            sum = rows_sum(sum);
            if (g == 0) part[wave * kpr + k * LCH + 16 * rt + n16] = m > -INFINITY ? m + __log2f(sum) : -INFINITY;
        }
        if (k + 1 < nch) chunk_stash<T, D>(cr, tiles + (size_t)((k + 1) & 1) * LCH * RW);
        if (k + 2 < nch) chunk_fetch<T, D>(cr, cb, ids, LCH * (k + 2));
        __syncthreads();
    }

    // ------------------------------------------- target, student, KL, dI
    // a2[s] = log2 of the teacher mass of slot s (combined over the waves)
    const float* sc = p.score + row * p.kp;
    float mt = -INFINITY, ms = -INFINITY;
    for (int s = threadIdx.x; s < nch * LCH; s += NT) {
        float a2 = -INFINITY;
        if (ids[s] >= 0) {
            const float l0 = part[s], l1 = part[kpr + s], l2 = part[2 * kpr + s], l3 = part[3 * kpr + s];
            const float M = fmaxf(fmaxf(l0, l1), fmaxf(l2, l3));
            a2 = M + __log2f((fast_exp2(l0 - M) + fast_exp2(l1 - M)) + (fast_exp2(l2 - M) + fast_exp2(l3 - M)));
            mt = fmaxf(mt, a2);
            ms = fmaxf(ms, sc[s]);
        }
        part[s] = a2;
    }
    mt = block_max(mt, red);
    ms = block_max(ms, red);
    float zt = 0.f, zs = 0.f;
    for (int s = threadIdx.x; s < nch * LCH; s += NT) {
        if (ids[s] >= 0) {
            zt += fast_exp2(part[s] - mt);
            zs += fast_exp2((sc[s] - ms) * LOG2E);
        }
    }
    zt = block_sum(zt, red);
    zs = block_sum(zs, red);
    const float lzt = __logf(zt), lzs = __logf(zs), izt = 1.f / zt, izs = 1.f / zs;
    const float dkl = grads ? p.dkl[row] : 0.f;
    float klp = 0.f;
    float* dI = part + kpr;                                    // dI per slot (pass 2 reads it)
    for (int s = threadIdx.x; s < kpr; s += NT) {
        float gi = 0.f;
        if (s < nch * LCH && ids[s] >= 0) {
            const float tg = fast_exp2(part[s] - mt) * izt;
            const float lt = (part[s] - mt) * LN2 - lzt;       // log target
            const float lp = (sc[s] - ms) - lzs;               // log student
            if (tg > 0.f) klp += tg * (lt - lp);
            gi = dkl * (__expf(sc[s] - ms) * izs - tg);
        }
        dI[s] = gi;
        if (grads && s < p.kp) gws[row * p.kp + s] = gi;
    }
    const float kl = block_sum(klp, red);                      // also orders the dI writes before pass 2
    if (p.kl && threadIdx.x == 0) p.kl[row] = nch > 0 ? kl : 0.f;
    if (!grads) return;

    // ---------------------------------------------- pass 2: student backward
    const int hh = 16 * wave + n16;                            // this lane's indexer head
    Frag<T> qif[KSI];
    const T* qirow = (const T*)p.qi + row * p.HI * DI;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qif[ks] = hh < p.HI ? load_frag(qirow + hh * DI + 32 * ks + 8 * g) : zero_frag<T>();
    const float wv = hh < p.HI ? p.w[row * p.HI + hh] : 0.f;
    f32x4 o[DTI];
#pragma unroll
    for (int dt = 0; dt < DTI; ++dt) o[dt] = f4zero();
    float dwl = 0.f;
    const T* kb = (const T*)p.ki + (int64_t)bi * p.nc * DI;
    piece_t kr[chunk_np<T, DI>()];
    if (nch > 0) { chunk_fetch<T, DI>(kr, kb, ids, 0); chunk_stash<T, DI>(kr, tiles); }
    if (nch > 1) chunk_fetch<T, DI>(kr, kb, ids, LCH);
    __syncthreads();
    for (int k = 0; k < nch; ++k) {
        const T* tile = tiles + (size_t)(k & 1) * LCH * RW;
        Frag<T> gb;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            // a^T[r, h] for 16 rows (m) and the wave's 16 heads (n)
            f32x4 a = f4zero();
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) a = mfma16(tile_frag<T, DI>(tile, 16 * rt + n16, ks, g), qif[ks], a);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gi = dI[k * LCH + 16 * rt + 4 * g + i];
                const bool pos = a[i] > 0.f;
                dwl += pos ? gi * a[i] : 0.f;
                gb.v[4 * rt + i] = from_f32<T>(pos ? gi * wv : 0.f);
            }
        }
        // dq_i^T[d, h] += sum_r K[r, d] G^T[r, h]
#pragma unroll
        for (int dt = 0; dt < DTI; ++dt) o[dt] = mfma16(rows_operand<T>(tile, DI, 0, 16 * dt, true), gb, o[dt]);
        if (k + 1 < nch) chunk_stash<T, DI>(kr, tiles + (size_t)((k + 1) & 1) * LCH * RW);
        if (k + 2 < nch) chunk_fetch<T, DI>(kr, kb, ids, LCH * (k + 2));
        __syncthreads();
    }
    dwl = rows_sum(dwl);
    if (hh < p.HI) {
        if (g == 0) p.dw[row * p.HI + hh] = dwl;
        T* dst = (T*)p.dqi + (row * p.HI + hh) * DI;
#pragma unroll
        for (int dt = 0; dt < DTI; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[16 * dt + 4 * g + i] = from_f32<T>(o[dt][i]);
    }
}

// ------------------------------------------------ dense warm-up, per query
// Contiguous rows j0 .. j0 + LCH - 1 of a [rows, W] matrix (rows past the
// last, jmax, read row jmax: their results are masked).
template <typename T, int W>
__device__ __forceinline__ void rows_fetch(piece_t* r, const T* base, int j0, int jmax)
{
    constexpr int PPR = chunk_ppr<T, W>(), NP = chunk_np<T, W>(), E16 = 16 / (int)sizeof(T);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int pc = (int)threadIdx.x + NT * k;
        const int rr = min(pc / PPR, LCH - 1), pp = pc % PPR;
        r[k] = *reinterpret_cast<const piece_t*>(base + (int64_t)min(j0 + rr, jmax) * W + pp * E16);
    }
}

// Dense warm-up form: the support of query t is every valid block j <
// n_valid(t).  One workgroup per query of the launch's chunk, teacher heads
// and indexer heads split 16 per wave.  Pass 1 walks the blocks in chunks of
// 32 (c rows and k_i rows in double-buffered LDS tiles), forms each wave's
// per-block log2 teacher mass and its part of the student score
// I = sum_h w_h relu(a_h); the waves' parts are combined by the thread that
// owns the block (thread j mod 256) and written to the query's two workspace
// rows (A: log2 mass, I: score; dense_ld floats each).  The owners then form
// the target / student statistics, the KL and dI (over A), reading back only
// what they wrote themselves.  Pass 2 (gradients) walks the k_i rows again
// as the selected form's pass 2 does, with dI handed over through LDS.
template <typename T, int D, int DI>
__global__ __launch_bounds__(NT) void loss_dense_query_kernel(LossArgs p, float* __restrict__ rows)
{
    constexpr int KS = D / 32, KSI = DI / 32, DTI = DI / 16;
    constexpr int CB = LCH * D * (int)sizeof(T), KB = LCH * DI * (int)sizeof(T);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T* ct = reinterpret_cast<T*>(smem);                          // [2][LCH][D] c rows
    T* kt = reinterpret_cast<T*>(smem + 2 * CB);                 // [2][LCH][DI] k_i rows
    float* tpart = reinterpret_cast<float*>(smem + 2 * CB + 2 * KB);   // [2][4][LCH] per-wave log2 masses
    float* spart = tpart + 2 * 4 * LCH;                          // [2][4][LCH] per-wave student parts
    float* dib = spart + 2 * 4 * LCH;                            // [2][LCH] dI of a chunk (pass 2)
    float* red = dib + 2 * LCH;                                  // [4]
    const int wave = threadIdx.x / WAVE, lane = lane_id(), g = lane / 16, n16 = lane % 16;
    const int bi = blockIdx.y;
    const int tl = p.t_count - 1 - (int)blockIdx.x;              // latest queries (most blocks) first
    const int t = p.t_begin + tl;
    const int64_t row = (int64_t)bi * p.S + t;
    float* arow = rows + ((int64_t)bi * p.t_count + tl) * 2 * p.dense_ld;
    float* irow = arow + p.dense_ld;
    const int nv = min((t + 1) / p.r, p.nc);
    const int nch = (nv + LCH - 1) / LCH;
    const bool grads = p.dqi != nullptr;
    const int owner = (int)threadIdx.x / LCH, oi = (int)threadIdx.x % LCH;   // blocks j = 256 m + threadIdx.x

    // ------------------------------------------ pass 1: teacher and student
    const T* qrow = (const T*)p.q + row * p.H * D;
    const T* qirow = (const T*)p.qi + row * p.HI * DI;
    const int hh = 16 * wave + n16;                              // A-row head of this lane
    Frag<T> qf[KS], qif[KSI];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = hh < p.H ? load_frag(qrow + hh * D + 32 * ks + 8 * g) : zero_frag<T>();
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qif[ks] = hh < p.HI ? load_frag(qirow + hh * DI + 32 * ks + 8 * g) : zero_frag<T>();
    float lse2[4], w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 16 * wave + 4 * g + i;                     // result-row head of element i
        lse2[i] = h < p.H ? p.lse[row * p.H + h] * LOG2E : INFINITY;   // +inf: padded heads add nothing
        w4[i] = h < p.HI ? p.w[row * p.HI + h] : 0.f;
    }
    const float sl2 = p.scale * LOG2E;
    const T* cb = (const T*)p.c + (int64_t)bi * p.nc * D;
    const T* kb = (const T*)p.ki + (int64_t)bi * p.nc * DI;
    const int jmax = max(p.nc - 1, 0);
    piece_t cr[chunk_np<T, D>()], kr[chunk_np<T, DI>()];
    if (nch > 0) {
        rows_fetch<T, D>(cr, cb, 0, jmax); chunk_stash<T, D>(cr, ct);
        rows_fetch<T, DI>(kr, kb, 0, jmax); chunk_stash<T, DI>(kr, kt);
    }
    if (nch > 1) { rows_fetch<T, D>(cr, cb, LCH, jmax); rows_fetch<T, DI>(kr, kb, LCH, jmax); }
    __syncthreads();
    for (int k = 0; k < nch; ++k) {
        const T* ctile = ct + (size_t)(k & 1) * LCH * D;
        const T* ktile = kt + (size_t)(k & 1) * LCH * DI;
        float* tp = tpart + (k & 1) * 4 * LCH;
        float* sp = spart + (k & 1) * 4 * LCH;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            // S[h, r] for the wave's 16 heads (m) and 16 rows (n); log2 mass over the heads
            f32x4 acc = f4zero();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma16(qf[ks], tile_frag<T, D>(ctile, 16 * rt + n16, ks, g), acc);
            float x[4];
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = fmaf(acc[i], sl2, -lse2[i]);
                m = fmaxf(m, x[i]);
            }
            m = rows_max(m);
            float sum = 0.f;
            if (m > -INFINITY) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sum += fast_exp2(x[i] - m);
            }
            sum = rows_sum(sum);
            // a[h, r] of the wave's 16 indexer heads; the weighted ReLU sum over them
            f32x4 a = f4zero();
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) a = mfma16(qif[ks], tile_frag<T, DI>(ktile, 16 * rt + n16, ks, g), a);
            float sv = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sv += w4[i] * fmaxf(a[i], 0.f);
            sv = rows_sum(sv);
            if (g == 0) {
                tp[wave * LCH + 16 * rt + n16] = m > -INFINITY ? m + __log2f(sum) : -INFINITY;
                sp[wave * LCH + 16 * rt + n16] = sv;
            }
        }
        if (k + 1 < nch) {
            chunk_stash<T, D>(cr, ct + (size_t)((k + 1) & 1) * LCH * D);
            chunk_stash<T, DI>(kr, kt + (size_t)((k + 1) & 1) * LCH * DI);
        }
        if (k + 2 < nch) {
            rows_fetch<T, D>(cr, cb, LCH * (k + 2), jmax);
            rows_fetch<T, DI>(kr, kb, LCH * (k + 2), jmax);
        }
        __syncthreads();
        // the owners of chunk k combine its four wave parts (the next write of
        // these parts comes after the next barrier)
        if (owner == (k & 7)) {
            const int j = k * LCH + oi;
            if (j < nv) {
                const float l0 = tp[oi], l1 = tp[LCH + oi], l2 = tp[2 * LCH + oi], l3 = tp[3 * LCH + oi];
                const float M = fmaxf(fmaxf(l0, l1), fmaxf(l2, l3));
                arow[j] = M > -INFINITY ? M + __log2f((fast_exp2(l0 - M) + fast_exp2(l1 - M)) +
                                                      (fast_exp2(l2 - M) + fast_exp2(l3 - M)))
                                        : -INFINITY;
                irow[j] = (sp[oi] + sp[LCH + oi]) + (sp[2 * LCH + oi] + sp[3 * LCH + oi]);
            }
        }
    }

    // ------------------------------------------- target, student, KL, dI
    float mt = -INFINITY, ms = -INFINITY;
    for (int j = threadIdx.x; j < nv; j += NT) {
        mt = fmaxf(mt, arow[j]);
        ms = fmaxf(ms, irow[j]);
    }
    mt = block_max(mt, red);
    ms = block_max(ms, red);
    float zt = 0.f, zs = 0.f;
    for (int j = threadIdx.x; j < nv; j += NT) {
        zt += fast_exp2(arow[j] - mt);
        zs += __expf(irow[j] - ms);
    }
    zt = block_sum(zt, red);
    zs = block_sum(zs, red);
    const float lzt = __logf(zt), lzs = __logf(zs), izt = 1.f / zt, izs = 1.f / zs;
    const float dkl = grads ? p.dkl[row] : 0.f;
    float klp = 0.f;
    for (int j = threadIdx.x; j < nv; j += NT) {
        const float a2 = arow[j], sc = irow[j];
        const float tg = fast_exp2(a2 - mt) * izt;
        const float lt = (a2 - mt) * LN2 - lzt;                  // log target
        const float lp = (sc - ms) - lzs;                        // log student
        if (tg > 0.f) klp += tg * (lt - lp);
        arow[j] = dkl * (__expf(sc - ms) * izs - tg);            // dI (read by the keys kernel)
    }
    const float kl = block_sum(klp, red);
    if (p.kl && threadIdx.x == 0) p.kl[row] = nch > 0 ? kl : 0.f;
    if (!grads) return;

    // ---------------------------------------------- pass 2: student backward
    const float wv = hh < p.HI ? p.w[row * p.HI + hh] : 0.f;
    f32x4 o[DTI];
#pragma unroll
    for (int dt = 0; dt < DTI; ++dt) o[dt] = f4zero();
    float dwl = 0.f;
    // the owners of chunk k hand its dI over to every wave through LDS
    auto hand = [&](int k) {
        if (owner == (k & 7)) {
            const int j = k * LCH + oi;
            dib[(k & 1) * LCH + oi] = j < nv ? arow[j] : 0.f;
        }
    };
    if (nch > 0) { rows_fetch<T, DI>(kr, kb, 0, jmax); chunk_stash<T, DI>(kr, kt); hand(0); }
    if (nch > 1) rows_fetch<T, DI>(kr, kb, LCH, jmax);
    __syncthreads();
    for (int k = 0; k < nch; ++k) {
        const T* tile = kt + (size_t)(k & 1) * LCH * DI;
        const float* dk = dib + (k & 1) * LCH;
        Frag<T> gb;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            // a^T[r, h] for 16 rows (m) and the wave's 16 heads (n)
            f32x4 a = f4zero();
#pragma unroll
            for (int ks = 0; ks < KSI; ++ks) a = mfma16(tile_frag<T, DI>(tile, 16 * rt + n16, ks, g), qif[ks], a);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gi = dk[16 * rt + 4 * g + i];
                const bool pos = a[i] > 0.f;
                dwl += pos ? gi * a[i] : 0.f;
                gb.v[4 * rt + i] = from_f32<T>(pos ? gi * wv : 0.f);
            }
        }
        // dq_i^T[d, h] += sum_r K[r, d] G^T[r, h]
#pragma unroll
        for (int dt = 0; dt < DTI; ++dt) o[dt] = mfma16(rows_operand<T>(tile, DI, 0, 16 * dt, true), gb, o[dt]);
        if (k + 1 < nch) { chunk_stash<T, DI>(kr, kt + (size_t)((k + 1) & 1) * LCH * DI); hand(k + 1); }
        if (k + 2 < nch) rows_fetch<T, DI>(kr, kb, LCH * (k + 2), jmax);
        __syncthreads();
    }
    dwl = rows_sum(dwl);
    if (hh < p.HI) {
        if (g == 0) p.dw[row * p.HI + hh] = dwl;
        T* dst = (T*)p.dqi + (row * p.HI + hh) * DI;
#pragma unroll
        for (int dt = 0; dt < DTI; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[16 * dt + 4 * g + i] = from_f32<T>(o[dt][i]);
    }
}

// ------------------------------------------------------ dk_i, key-stationary
struct KeysGeom {
    int Qb, nqb, ntiles;
};

// DENSE: every valid block is the support; the query's dI row (dense_ld
// floats, chunk-local) is read directly instead of through its index row.
template <typename T, int DI, bool DENSE>
__global__ __launch_bounds__(NT) void loss_keys_kernel(LossArgs p, KeysGeom geo, const float* __restrict__ gws,
                                                       float* __restrict__ part)
{
    constexpr int KSI = DI / 32, DTI = DI / 16, RT = KRW / 16, HP = 64;
    constexpr int QPIECES = HP * DI * (int)sizeof(T) / 16;    // 16-byte pieces of one query's q_i tile
    constexpr int NPQ = (QPIECES + NT - 1) / NT;
    constexpr int E16 = 16 / (int)sizeof(T);
    constexpr int IPT = 2048 / NT;                             // index entries per thread, K' <= 2048
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T* qt = reinterpret_cast<T*>(smem);                        // [2][HP][DI] q_i, rows = heads, swizzled
    float* wt = reinterpret_cast<float*>(qt + 2 * HP * DI);    // [2][HP]
    float* gt = wt + 2 * HP;                                   // [3][KTR] dI of the tile's rows for one query
    const int wave = threadIdx.x / WAVE, lane = lane_id(), g = lane / 16, n16 = lane % 16;

    // the tiles of one query block run on one XCD (workgroups are dealt to
    // the 8 XCDs round robin), so its q_i stays in that XCD's L2
    const int lin = blockIdx.x;
    const int group = lin / (8 * geo.ntiles), rem = lin % (8 * geo.ntiles);
    const int qbi = group * 8 + rem % 8, tile = rem / 8;
    if (qbi >= p.b * geo.nqb) return;
    const int bi = qbi / geo.nqb, qb = geo.nqb - 1 - qbi % geo.nqb;
    const int tile_lo = tile * KTR;
    const int tb = p.t_begin, te = p.t_begin + p.t_count;
    const int t0 = max(tb + qb * geo.Qb, (tile_lo + 1) * p.r - 1);
    const int t1 = min(te, tb + (qb + 1) * geo.Qb);
    if (t0 >= t1) return;                                       // no query of the block reaches the tile
    const int hp_n = (p.HI + 31) / 32;                          // 32-head pairs in use

    // this wave's k_i rows as B operands (n = row, k = d)
    Frag<T> kf[RT][KSI];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int j = tile_lo + wave * KRW + 16 * rt + n16;
        const T* src = (const T*)p.ki + ((int64_t)bi * p.nc + (j < p.nc ? j : 0)) * DI;
#pragma unroll
        for (int ks = 0; ks < KSI; ++ks) kf[rt][ks] = j < p.nc ? load_frag(src + 32 * ks + 8 * g) : zero_frag<T>();
    }
    f32x4 acc[DTI][RT];
#pragma unroll
    for (int dt = 0; dt < DTI; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[dt][rt] = f4zero();

    piece_t qreg[NPQ];
    float wreg = 0.f;
    int jreg[IPT];
    float greg[IPT];
    auto prefetch = [&](int t) {
        const int64_t row = (int64_t)bi * p.S + t;
        const T* qsrc = (const T*)p.qi + row * p.HI * DI;
#pragma unroll
        for (int k = 0; k < NPQ; ++k) {
            const int pc = (int)threadIdx.x + NT * k;
            const int h = pc / (DI / E16);
            if (pc < QPIECES) qreg[k] = h < p.HI ? *reinterpret_cast<const piece_t*>(qsrc + (int64_t)pc * E16)
                                                 : piece_t{0u, 0u, 0u, 0u};
        }
        if (threadIdx.x < HP) wreg = (int)threadIdx.x < p.HI ? p.w[row * p.HI + threadIdx.x] : 0.f;
        if constexpr (DENSE) {
            const int j = tile_lo + (int)threadIdx.x, nvt = min((t + 1) / p.r, p.nc);
            greg[0] = ((int)threadIdx.x < KTR && j < nvt)
                          ? gws[((int64_t)bi * p.t_count + (t - tb)) * 2 * p.dense_ld + j] : 0.f;
        } else {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int s = (int)threadIdx.x + NT * k;
                jreg[k] = s < p.kp ? p.idx[row * p.kp + s] : -1;
                greg[k] = s < p.kp ? gws[row * p.kp + s] : 0.f;
            }
        }
    };
    auto place = [&](int buf, int cb) {
        T* dst = qt + (size_t)buf * HP * DI;
#pragma unroll
        for (int k = 0; k < NPQ; ++k) {
            const int pc = (int)threadIdx.x + NT * k;
            if (pc < QPIECES) {
                const int h = pc / (DI / E16), pos = (pc % (DI / E16)) * E16;
                *reinterpret_cast<piece_t*>(dst + h * DI + ((((pos >> 3) ^ unit_swz(h, DI / 8))) << 3) + (pos & 7)) =
                    qreg[k];
            }
        }
        if (threadIdx.x < HP) wt[buf * HP + threadIdx.x] = wreg;
        float* gtb = gt + cb * KTR;
        if constexpr (DENSE) {
            if ((int)threadIdx.x < KTR) gtb[threadIdx.x] = greg[0];
        } else {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int j = jreg[k] - tile_lo;
                if (j >= 0 && j < KTR && greg[k] != 0.f) atomicAdd(&gtb[j], greg[k]);
            }
        }
    };

    for (int i = threadIdx.x; i < 3 * KTR; i += NT) gt[i] = 0.f;
    __syncthreads();
    prefetch(t0);
    place(0, 0);
    if (t0 + 1 < t1) prefetch(t0 + 1);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
        const int k = t - t0, buf = k & 1, cb = k % 3;
        const T* qtile = qt + (size_t)buf * HP * DI;
        const float* wb = wt + buf * HP;
        float gj[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) gj[rt] = gt[cb * KTR + wave * KRW + 16 * rt + n16];
        for (int hp = 0; hp < hp_n; ++hp) {
            Frag<T> gb[RT];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int ht = 2 * hp + h2;
                Frag<T> af[KSI];
#pragma unroll
                for (int ks = 0; ks < KSI; ++ks) af[ks] = tile_frag<T, DI>(qtile, 16 * ht + n16, ks, g);
                float wv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) wv[i] = wb[16 * ht + 4 * g + i];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    // a[h, j] for 16 heads (m) and 16 rows (n)
                    f32x4 a = f4zero();
#pragma unroll
                    for (int ks = 0; ks < KSI; ++ks) a = mfma16(af[ks], kf[rt][ks], a);
#pragma unroll
                    for (int i = 0; i < 4; ++i) gb[rt].v[4 * h2 + i] = from_f32<T>(a[i] > 0.f ? gj[rt] * wv[i] : 0.f);
                }
            }
            // dk_i^T[d, j] += sum_h q_i[h, d] G[h, j]
#pragma unroll
            for (int dt = 0; dt < DTI; ++dt) {
                const Frag<T> qa = rows_operand<T>(qtile, DI, 32 * hp, 16 * dt, true);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[dt][rt] = mfma16(qa, gb[rt], acc[dt][rt]);
            }
        }
        if (t + 1 < t1) place(buf ^ 1, (k + 1) % 3);
        {
            float* nxt = gt + ((k + 2) % 3) * KTR;              // used two queries ago; next filled one query on
            for (int i = threadIdx.x; i < KTR; i += NT) nxt[i] = 0.f;
        }
        if (t + 2 < t1) prefetch(t + 2);
        __syncthreads();
    }
    float* dst = part + (((int64_t)bi * geo.nqb + qb) * p.nc) * DI;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int j = tile_lo + wave * KRW + 16 * rt + n16;
        if (j < p.nc) {
#pragma unroll
            for (int dt = 0; dt < DTI; ++dt)
                *reinterpret_cast<f32x4*>(dst + (int64_t)j * DI + 16 * dt + 4 * g) = acc[dt][rt];
        }
    }
}

// dk_i[b, j, :] = sum over query blocks that reach block j of their partial
// rows.  A workgroup takes 64 consecutive float4 columns of the output and
// splits the query blocks of each over 4 lanes (block q to lane q % 4); the
// four partial sums are then added in lane order, so the order is fixed.
__global__ __launch_bounds__(NT) void loss_reduce_kernel(LossArgs p, KeysGeom geo, const float* __restrict__ part)
{
    __shared__ f32x4 red[4][64];
    const int col = threadIdx.x % 64, split = threadIdx.x / 64;
    const int v4 = p.DI / 4;
    const int64_t i = (int64_t)blockIdx.x * 64 + col;   // one float4 of one row
    const bool live = i < (int64_t)p.b * p.nc * v4;
    f32x4 s = f4zero();
    int64_t bj = 0;
    int v = 0;
    if (live) {
        v = (int)(i % v4);
        bj = i / v4;
        const int j = (int)(bj % p.nc), bi = (int)(bj / p.nc);
        const int qlo = max(0, ((j + 1) * p.r - 1 - p.t_begin) / geo.Qb);
        for (int q = qlo + split; q < geo.nqb; q += 4)
            s += *reinterpret_cast<const f32x4*>(part + ((((int64_t)bi * geo.nqb + q) * p.nc) + j) * p.DI + 4 * v);
    }
    red[split][col] = s;
    __syncthreads();
    if (split == 0 && live) {
        f32x4* dst = reinterpret_cast<f32x4*>(p.dki + bj * p.DI + 4 * v);
        const f32x4 sum = ((red[0][col] + red[1][col]) + red[2][col]) + red[3][col];
        *dst = p.dk_accumulate ? *dst + sum : sum;
    }
}

// qb > 0: that query block (the dense plan's); else the smallest power of
// two from 32 that keeps the partial rows within 1 GiB
KeysGeom keys_geometry(const LossArgs& p, int qb = 0)
{
    KeysGeom g{};
    auto part_bytes = [&](int q) { return (int64_t)p.b * ((p.t_count + q - 1) / q) * p.nc * p.DI * 4; };
    if (qb <= 0) {
        qb = 32;
        while (qb < 4096 && part_bytes(qb) > ((int64_t)1 << 30)) qb *= 2;
    }
    g.Qb = qb;
    g.nqb = (p.t_count + qb - 1) / qb;
    g.ntiles = (p.nc + KTR - 1) / KTR;
    return g;
}

int64_t gws_floats(const LossArgs& p) { return ((int64_t)p.b * p.S * p.kp + 63) / 64 * 64; }

template <typename T, int D, int DI>
hipError_t launch_loss(const LossArgs& p, float* ws, hipStream_t st)
{
    constexpr int RW = D > DI ? D : DI;
    const int kpr = (p.kp + LCH - 1) / LCH * LCH;
    const size_t lds = 2 * (size_t)LCH * RW * sizeof(T) + (size_t)kpr * (4 * 4 + 4) + 16;
    if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    auto qk = loss_query_kernel<T, D, DI>;
    hipError_t e = hipFuncSetAttribute((const void*)qk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    {
        TimedLaunch tl(K_LOSS_QUERY, st);
        hipLaunchKernelGGL(qk, dim3(p.S, p.b), dim3(NT), lds, st, p, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!p.dqi || p.nc == 0 || p.kp == 0) return hipSuccess;   // no block: dk_i has no rows
    const KeysGeom geo = keys_geometry(p);
    float* part = ws + gws_floats(p);
    const size_t klds = 2 * (size_t)64 * DI * sizeof(T) + 2 * 64 * 4 + 3 * KTR * 4;
    auto kk = loss_keys_kernel<T, DI, false>;
    if ((e = hipFuncSetAttribute((const void*)kk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)klds)) != hipSuccess)
        return e;
    const int64_t groups = ((int64_t)p.b * geo.nqb + 7) / 8;
    {
        TimedLaunch tl(K_LOSS_KEYS, st);
        hipLaunchKernelGGL(kk, dim3((unsigned)(groups * 8 * geo.ntiles)), dim3(NT), klds, st, p, geo, ws, part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t cols = (int64_t)p.b * p.nc * (p.DI / 4);
    {
        TimedLaunch tl(K_LOSS_REDUCE, st);
        hipLaunchKernelGGL(loss_reduce_kernel, dim3((unsigned)((cols + 63) / 64)), dim3(NT), 0, st, p, geo, part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int D>
hipError_t loss_di(const LossArgs& p, float* ws, hipStream_t st)
{
    switch (p.DI) {
    case 32: return launch_loss<T, D, 32>(p, ws, st);
    case 64: return launch_loss<T, D, 64>(p, ws, st);
    case 128: return launch_loss<T, D, 128>(p, ws, st);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------ dense warm-up: the plan
// The queries run in chunks of qc (a multiple of the keys kernel's query
// block); per chunk the workspace holds each query's two rows (dense_ld
// floats each: log2 teacher mass, then dI; student scores) and the chunk's
// dk_i partial rows.  The plan takes the largest chunk whose bytes fit the
// budget, so memory is O(budget), never O(sq * n_c) unless the budget allows.
constexpr int DENSE_QB = 32;

int dense_ld(const LossArgs& p) { return (max(p.nc, 1) + LCH - 1) / LCH * LCH; }

int64_t dense_rows_floats(const LossArgs& p, int qc)
{
    return ((int64_t)p.b * qc * 2 * dense_ld(p) + 63) / 64 * 64;   // partial rows start 256-byte aligned
}

int64_t dense_bytes(const LossArgs& p, int qc)
{
    const int64_t part = (int64_t)p.b * ((qc + DENSE_QB - 1) / DENSE_QB) * p.nc * p.DI;
    return (dense_rows_floats(p, qc) + part) * (int64_t)sizeof(float);
}

int dense_chunk(const LossArgs& p, size_t budget)
{
    int lo = 1, hi = (p.S + DENSE_QB - 1) / DENSE_QB;               // chunk sizes in query blocks
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (dense_bytes(p, mid * DENSE_QB) <= (int64_t)budget) lo = mid;
        else hi = mid - 1;
    }
    return lo * DENSE_QB;
}

template <typename T, int D, int DI>
hipError_t launch_dense(const LossArgs& p0, float* ws, int qc, hipStream_t st)
{
    constexpr int CB = LCH * D * (int)sizeof(T), KB = LCH * DI * (int)sizeof(T);
    const size_t lds = 2 * (size_t)CB + 2 * (size_t)KB + (2 * 4 * LCH * 2 + 2 * LCH + 4) * sizeof(float);
    if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    auto qk = loss_dense_query_kernel<T, D, DI>;
    hipError_t e = hipFuncSetAttribute((const void*)qk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    auto kk = loss_keys_kernel<T, DI, true>;
    const size_t klds = 2 * (size_t)64 * DI * sizeof(T) + 2 * 64 * 4 + 3 * KTR * 4;
    if ((e = hipFuncSetAttribute((const void*)kk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)klds)) != hipSuccess)
        return e;
    const bool grads = p0.dqi != nullptr;
    float* part = ws + dense_rows_floats(p0, qc);
    for (int t0 = 0; t0 < p0.S; t0 += qc) {
        LossArgs p = p0;
        p.t_begin = t0;
        p.t_count = min(qc, p0.S - t0);
        p.dense_ld = dense_ld(p0);
        p.dk_accumulate = t0 > 0;
        {
            TimedLaunch tl(K_LOSS_QUERY, st);
            hipLaunchKernelGGL(qk, dim3(p.t_count, p.b), dim3(NT), lds, st, p, ws);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (!grads || p.nc == 0) continue;
        const KeysGeom geo = keys_geometry(p, DENSE_QB);
        const int64_t groups = ((int64_t)p.b * geo.nqb + 7) / 8;
        {
            TimedLaunch tl(K_LOSS_KEYS, st);
            hipLaunchKernelGGL(kk, dim3((unsigned)(groups * 8 * geo.ntiles)), dim3(NT), klds, st, p, geo,
                               (const float*)ws, part);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const int64_t cols = (int64_t)p.b * p.nc * (p.DI / 4);
        {
            TimedLaunch tl(K_LOSS_REDUCE, st);
            hipLaunchKernelGGL(loss_reduce_kernel, dim3((unsigned)((cols + 63) / 64)), dim3(NT), 0, st, p, geo, part);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <typename T, int D>
hipError_t dense_di(const LossArgs& p, float* ws, int qc, hipStream_t st)
{
    switch (p.DI) {
    case 32: return launch_dense<T, D, 32>(p, ws, qc, st);
    case 64: return launch_dense<T, D, 64>(p, ws, qc, st);
    case 128: return launch_dense<T, D, 128>(p, ws, qc, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t indexer_loss_dense_workspace_bytes(const LossArgs& p, size_t budget)
{
    return (size_t)dense_bytes(p, dense_chunk(p, budget));
}

hipError_t indexer_loss_dense(const LossArgs& p, bool bf16, float* ws, size_t ws_bytes, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    const int qc = dense_chunk(p, ws_bytes);
    if (bf16) {
        switch (p.D) {
        case 64: return dense_di<bf16_t, 64>(p, ws, qc, st);
        case 128: return dense_di<bf16_t, 128>(p, ws, qc, st);
        case 512: return dense_di<bf16_t, 512>(p, ws, qc, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.D) {
    case 64: return dense_di<float, 64>(p, ws, qc, st);
    case 128: return dense_di<float, 128>(p, ws, qc, st);
    default: return hipErrorInvalidValue;
    }
}

size_t indexer_loss_workspace_bytes(const LossArgs& p)
{
    const KeysGeom g = keys_geometry(p);
    return (size_t)(gws_floats(p) + (int64_t)p.b * g.nqb * p.nc * p.DI) * sizeof(float);
}

hipError_t indexer_loss(const LossArgs& p, bool bf16, float* ws, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    if (bf16) {
        switch (p.D) {
        case 64: return loss_di<bf16_t, 64>(p, ws, st);
        case 128: return loss_di<bf16_t, 128>(p, ws, st);
        case 512: return loss_di<bf16_t, 512>(p, ws, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.D) {
    case 64: return loss_di<float, 64>(p, ws, st);
    case 128: return loss_di<float, 128>(p, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csa
