// index_topk.hip -- learned indexer scores + streaming top-k (gfx950).
//
//   I[t, j] = sum_h w[t, h] * relu(q_i[t, h] . k_i[j]),   j < n_valid(t) = (t+1)/ratio
//
// Megatron-LM PR #7152 (min-memory DSA kernels): scores are produced and
// reduced tile by tile, so memory is O(tile) and the [sq, n_c] matrix never
// exists; one full top-k (not a merge of chunked top-ks) defines the result,
// with ties to the lower index; indices and scores leave ordered by position.
// Megatron-LM PR #6400 (causal-mask thread): block j is invalid for t iff
// j >= (t+1)//ratio, and rows with fewer valid blocks than K' are padded
// with -1.
//
// Work split: a workgroup is 4 waves = 4 consecutive queries of one batch.
// For each tile of 64 indexer keys the workgroup stages k_i into LDS; each
// wave multiplies its query's q_i (all heads, held in registers as MFMA A
// operands) against the tile: S[h, j] on 16x16x32 MFMA, ReLU, the per-head
// weights and the sum over heads stay in registers (in-lane plus two
// cross-lane adds), leaving lane l with the score of key j0 + l.
//
// Streaming top-k: each wave keeps a candidate buffer in LDS.  Keys arrive
// in ascending index, and a key is appended (ballot + mbcnt compaction) iff
// its score beats the current threshold tau; the buffer therefore stays
// sorted by index.  When the next tile could overflow it, the buffer is cut:
// first by keeping the value-histogram bin that holds the K'-th best and every
// bin above it (tau becomes the smallest kept score), or, when that bin holds
// too many entries, to exactly the K' best (tau becomes the K'-th score).
// Either way at least K' kept entries beat every dropped entry and every later
// key scoring at most tau (equal scores lose on their larger index), so
// nothing of the final top K' is lost.  The exact cut is a wave-level
// selection: value histograms over the current [lo, hi] range narrow down to
// one bin, which is ranked exactly; ties at the threshold are kept in buffer
// order, i.e. lowest index first.  At the end the exact selection keeps
// min(K', n_valid) entries and the buffer is written out as is: already in
// ascending index.
#include <cstdlib>

#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "timing.hpp"

namespace csa {

namespace {

constexpr int KT = 64;          // keys per tile
constexpr int HBINS = 256;      // histogram bins per selection level

}  // namespace

// LDS bytes of one workgroup: the key tile plus, per wave, the candidate
// buffer (score + index), a histogram and a 64-entry scratch.
size_t topk_lds_bytes(int DI, int elem, int cap)
{
    return (size_t)KT * (DI + 16 / elem) * elem + 4 * ((size_t)cap * 8 + HBINS * 4 + 64 * 8);
}

namespace {

struct WaveBufs {
    float* s;        // candidate scores   [cap]
    int* j;          // candidate indices  [cap]
    unsigned* hist;  // [HBINS]
    float* xs;       // small-set scratch  [64]
    int* xj;         // [64]
};

__device__ __forceinline__ int bin_of(float s, float lo, float scale)
{
    if (s <= lo) return 0;
    float f = fminf((s - lo) * scale, (float)(HBINS - 1));
    return (int)f;
}

// Each pass over the buffer reads SB entries per lane before it uses any of
// them, so that one pass waits for LDS about n / (64 SB) times, not n / 64
// (the kernels use SB = 8 in bf16, fewer in fp32, whose registers are fuller).

// s[u] (and j[u]) = entry i0 + 64 u + lane of the buffer, where it is < n
template <int SB>
__device__ __forceinline__ void read_batch(const WaveBufs& b, int i0, int n, float (&s)[SB])
{
    const int lane = lane_id();
#pragma unroll
    for (int u = 0; u < SB; ++u) {
        const int i = i0 + u * WAVE + lane;
        s[u] = i < n ? b.s[i] : -INFINITY;
    }
}
template <int SB>
__device__ __forceinline__ void read_batch(const WaveBufs& b, int i0, int n, float (&s)[SB], int (&j)[SB])
{
    const int lane = lane_id();
#pragma unroll
    for (int u = 0; u < SB; ++u) {
        const int i = i0 + u * WAVE + lane;
        s[u] = i < n ? b.s[i] : -INFINITY;
        j[u] = i < n ? b.j[i] : 0;
    }
}

// Keep the k best of b.s/b.j[0..n) by (score desc, index asc), preserving
// buffer order.  Requires 1 <= k < n.  Returns the threshold score T (the
// k-th best score).  Wave-uniform control flow.
template <int SB>
__device__ float select_keep(const WaveBufs& b, int n, int k)
{
    const int lane = lane_id();
    float lo = INFINITY, hi = -INFINITY;
    for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
        float s[SB];
        read_batch(b, i0, n, s);
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            if (i0 + u * WAVE + lane < n) {
                lo = fminf(lo, s[u]);
                hi = fmaxf(hi, s[u]);
            }
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    int kk = k;          // rank sought inside [lo, hi]
    float T = lo;
    int need = kk;       // ties at T to keep (in buffer order)
    for (int level = 0; level < 64; ++level) {
        if (!(hi > lo)) { T = lo; need = kk; break; }
        // histogram of the entries inside [lo, hi]
        for (int i = lane; i < HBINS; i += WAVE) b.hist[i] = 0u;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        const float scale = (float)HBINS / (hi - lo);
        for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
            float s[SB];
            read_batch(b, i0, n, s);
#pragma unroll
            for (int u = 0; u < SB; ++u)
                if (i0 + u * WAVE + lane < n && s[u] >= lo && s[u] <= hi) atomicAdd(&b.hist[bin_of(s[u], lo, scale)], 1u);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // suffix counts over lanes: lane l owns bins 4l..4l+3
        unsigned c0 = b.hist[4 * lane], c1 = b.hist[4 * lane + 1], c2 = b.hist[4 * lane + 2],
                 c3 = b.hist[4 * lane + 3];
        int mine = (int)(c0 + c1 + c2 + c3);
        int suf = mine;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            int v = __shfl_down(suf, o);
            if (lane + o < WAVE) suf += v;
        }
        uint64_t ge = __ballot(suf >= kk);
        int ls = 63 - __clzll((long long)ge);
        int above_lane = __shfl(suf - mine, ls);        // entries in bins above lane ls
        int cb[4] = {(int)__shfl((int)c0, ls), (int)__shfl((int)c1, ls), (int)__shfl((int)c2, ls),
                     (int)__shfl((int)c3, ls)};
        int cum = above_lane, bstar = 4 * ls, above_b = above_lane, cnt_b = cb[0];
#pragma unroll
        for (int q = 3; q >= 0; --q) {
            if (cum < kk && cum + cb[q] >= kk) { bstar = 4 * ls + q; above_b = cum; cnt_b = cb[q]; }
            cum += cb[q];
        }
        kk -= above_b;
        // range of the chosen bin
        float lo2 = INFINITY, hi2 = -INFINITY;
        for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
            float s[SB];
            read_batch(b, i0, n, s);
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                if (i0 + u * WAVE + lane < n && s[u] >= lo && s[u] <= hi && bin_of(s[u], lo, scale) == bstar) {
                    lo2 = fminf(lo2, s[u]);
                    hi2 = fmaxf(hi2, s[u]);
                }
            }
        }
        lo2 = wave_min(lo2);
        hi2 = wave_max(hi2);
        if (cnt_b <= WAVE) {
            // gather the bin's entries into lanes (in buffer order) and rank them exactly
            int base = 0;
            for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
                float s[SB];
                int jj[SB];
                read_batch(b, i0, n, s, jj);
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const bool in = i0 + u * WAVE + lane < n && s[u] >= lo2 && s[u] <= hi2;
                    const uint64_t m = __ballot(in);
                    if (in) {
                        const int p = base + (int)mbcnt(m);
                        b.xs[p] = s[u];
                        b.xj[p] = jj[u];
                    }
                    base += __popcll(m);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float ms = lane < cnt_b ? b.xs[lane] : -INFINITY;
            int mj = lane < cnt_b ? b.xj[lane] : 0x7fffffff;
            int rank = 0, gt = 0;
            for (int q = 0; q < cnt_b; ++q) {
                float os = __shfl(ms, q);
                int oj = __shfl(mj, q);
                rank += (os > ms || (os == ms && oj < mj)) ? 1 : 0;
                gt += os > ms ? 1 : 0;
            }
            uint64_t hit = __ballot(lane < cnt_b && rank == kk - 1);
            int lh = __ffsll((long long)hit) - 1;
            T = __shfl(ms, lh);
            int gtT = __shfl(gt, lh);       // entries of the bin strictly above T
            need = kk - gtT;
            break;
        }
        lo = lo2;
        hi = hi2;
    }
    // in-order compaction: a batch is read whole before any of it is written,
    // and an entry only moves down, so no write lands on an unread entry
    int out = 0, ties = 0;
    for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
        float s[SB];
        int jj[SB];
        read_batch(b, i0, n, s, jj);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const bool in = i0 + u * WAVE + lane < n;
            const bool eq = in && s[u] == T;
            const uint64_t em = __ballot(eq);
            const int tr = ties + (int)mbcnt(em);
            ties += __popcll(em);
            const bool keep = in && (s[u] > T || (eq && tr < need));
            const uint64_t km = __ballot(keep);
            if (keep) {
                const int p = out + (int)mbcnt(km);
                b.s[p] = s[u];
                b.j[p] = jj[u];
            }
            out += __popcll(km);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return T;
}

// A cut that only makes room (before the stream ends): keep every entry whose
// histogram bin over [lo, hi] (the buffer's score range) is at or above the
// bin holding the k-th best, if that keeps at most `limit` entries.  Every
// dropped entry then scores below every kept one, of which there are at least
// k, so none of them can reach the final k best; and a later key whose score
// is at most the smallest kept score (returned in tau) ranks below at least k
// kept entries with that score or more and lower indices, so it may be
// rejected too.  The exact selection at the end of the stream is unchanged.
// Returns the number kept, or 0 (buffer untouched) when the bin of the k-th
// best holds too many entries for the limit, or the range is empty.
template <int SB>
__device__ int select_room(const WaveBufs& b, int n, int k, int limit, float lo, float hi, float& tau)
{
    const int lane = lane_id();
    if (!(hi > lo)) return 0;
    for (int i = lane; i < HBINS; i += WAVE) b.hist[i] = 0u;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const float scale = (float)HBINS / (hi - lo);
    // every entry gets a bin (bin_of clamps), and bins are monotonic in the score
    for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
        float s[SB];
        read_batch(b, i0, n, s);
#pragma unroll
        for (int u = 0; u < SB; ++u)
            if (i0 + u * WAVE + lane < n) atomicAdd(&b.hist[bin_of(s[u], lo, scale)], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const unsigned c0 = b.hist[4 * lane], c1 = b.hist[4 * lane + 1], c2 = b.hist[4 * lane + 2],
                   c3 = b.hist[4 * lane + 3];
    const int mine = (int)(c0 + c1 + c2 + c3);
    int suf = mine;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int v = __shfl_down(suf, o);
        if (lane + o < WAVE) suf += v;
    }
    const int ls = 63 - __clzll((long long)__ballot(suf >= k));
    const int above_lane = __shfl(suf - mine, ls);
    const int cb[4] = {(int)__shfl((int)c0, ls), (int)__shfl((int)c1, ls), (int)__shfl((int)c2, ls),
                       (int)__shfl((int)c3, ls)};
    int cum = above_lane, bstar = 4 * ls, keep_n = 0;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
        if (cum < k && cum + cb[q] >= k) { bstar = 4 * ls + q; keep_n = cum + cb[q]; }
        cum += cb[q];
    }
    if (keep_n > limit) return 0;
    // in-order compaction, as in select_keep
    int out = 0;
    float mn = INFINITY;
    for (int i0 = 0; i0 < n; i0 += SB * WAVE) {
        float s[SB];
        int jj[SB];
        read_batch(b, i0, n, s, jj);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const bool keep = i0 + u * WAVE + lane < n && bin_of(s[u], lo, scale) >= bstar;
            const uint64_t km = __ballot(keep);
            if (keep) {
                const int p = out + (int)mbcnt(km);
                b.s[p] = s[u];
                b.j[p] = jj[u];
                mn = fminf(mn, s[u]);
            }
            out += __popcll(km);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    tau = wave_min(mn);
    return out;
}

// element strides: q_i (batch, token, head), k_i (batch, block), w (batch, token)
struct IndexStrides { int64_t qb, qs, qh, kb, ks, wb, ws; };

template <typename T, int DI, int HT>
__global__ __launch_bounds__(256, 2) void index_topk_kernel(const T* __restrict__ qi,
                                                            const T* __restrict__ ki,
                                                            const float* __restrict__ w,
                                                            const int32_t* __restrict__ doc,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ score, int S,
                                                            int HI, int r, int nc, int kp, int cap,
                                                            IndexStrides is)
{
    constexpr int KS = DI / 32;            // k-steps of 32
    // buffer entries per lane per read batch (fp32 at d_i = 128 with four head
    // tiles has no registers to spare)
    constexpr int SB = sizeof(T) == 2 ? 8 : (DI == 128 && HT == 4 ? 1 : 4);
    constexpr bool ROOM = !(sizeof(T) == 4 && DI == 128 && HT == 4);   // the loose cut (same registers)
    constexpr int ROW = DI + 16 / sizeof(T) * 1;   // LDS row stride (elements), one 16-B pad
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T* ktile = reinterpret_cast<T*>(smem);
    char* wbase = smem + (size_t)KT * ROW * sizeof(T);
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int g = lane / 16, n16 = lane % 16;
    const size_t per_wave = (size_t)cap * 8 + HBINS * 4 + 64 * 8;
    char* mine = wbase + per_wave * wave;
    WaveBufs bufs;
    bufs.s = reinterpret_cast<float*>(mine);
    bufs.j = reinterpret_cast<int*>(mine + (size_t)cap * 4);
    bufs.hist = reinterpret_cast<unsigned*>(mine + (size_t)cap * 8);
    bufs.xs = reinterpret_cast<float*>(mine + (size_t)cap * 8 + HBINS * 4);
    bufs.xj = reinterpret_cast<int*>(mine + (size_t)cap * 8 + HBINS * 4 + 64 * 4);

    const int bi = blockIdx.y;
    // latest queries (most valid blocks) first: short ones fill the tail
    const int qblk = (int)gridDim.x - 1 - (int)blockIdx.x;
    const int t = qblk * 4 + wave;
    const bool active = t < S;
    const int nv = active ? min((t + 1) / r, nc) : 0;
    const int t_last = min(qblk * 4 + 3, S - 1);
    const int nv_max = min((t_last + 1) / r, nc);
    const int64_t row = (int64_t)bi * S + (active ? t : 0);
    const T* qrow = qi + bi * is.qb + (int64_t)(active ? t : 0) * is.qs;
    const float* wrow = w ? w + bi * is.wb + (int64_t)(active ? t : 0) * is.ws : nullptr;

    // query operands (A: m = head, k = dim) and per-head weights in C-row layout
    Frag<T> qa[HT][KS];
    float wv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = 16 * ht + n16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qa[ht][ks] = (active && h < HI) ? load_frag(qrow + h * is.qh + 32 * ks + 8 * g) : zero_frag<T>();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 16 * ht + 4 * g + i;
            wv[ht][i] = (active && hh < HI) ? (w ? wrow[hh] : 1.f) : 0.f;   // no w: unit weights
        }
    }

    const T* kb = ki + bi * is.kb;
    float tau = -INFINITY;
    int cnt = 0;
    float rlo = INFINITY, rhi = -INFINITY;           // this lane's share of the buffer's score range
    // the loose cut may keep up to half the headroom above K' (tried only
    // when that leaves at least a tile's worth of slack)
    const int room_limit = kp + (cap - kp) / 2 - KT;
    const bool try_room = ROOM && room_limit >= kp + KT;
    constexpr int CH = 16 / sizeof(T);               // elements per 16-B chunk
    constexpr int CHUNKS = KT * DI / CH;
    constexpr int CPT = CHUNKS / 256;                // chunks per thread
    static_assert(CPT * 256 == CHUNKS, "a key tile splits evenly over the workgroup");
    // the next key tile is loaded into registers while the current one computes
    uint4 pre[CPT];
    // packed documents: block j belongs to the document of token j*r
    const int32_t* dcol = doc ? doc + (int64_t)bi * S : nullptr;
    const int dt = (dcol && active) ? dcol[t] : 0;
    int dpre = 0, dcur = 0;
    auto load_tile = [&](int j0) {
        if (dcol) dpre = j0 + lane < nc ? dcol[(j0 + lane) * r] : 0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int c = (int)threadIdx.x + 256 * k;
            const int rr = c / (DI / CH), cc = (c % (DI / CH)) * CH;
            pre[k] = j0 + rr < nc ? *reinterpret_cast<const uint4*>(kb + (int64_t)(j0 + rr) * is.ks + cc)
                                  : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    if (nv_max > 0) load_tile(0);
    for (int j0 = 0; j0 < nv_max; j0 += KT) {
        __syncthreads();                              // every wave is done with the previous tile
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int c = (int)threadIdx.x + 256 * k;
            const int rr = c / (DI / CH), cc = (c % (DI / CH)) * CH;
            *reinterpret_cast<uint4*>(ktile + rr * ROW + cc) = pre[k];
        }
        dcur = dpre;
        if (j0 + KT < nv_max) load_tile(j0 + KT);
        __syncthreads();
        if (j0 >= nv) continue;
        float my = -INFINITY;
        // bf16: the tile's 4 x KS key fragments are read before the first MFMA
        // (one LDS round trip per tile instead of one per fragment)
        constexpr bool EARLY = sizeof(T) == 2;
        Frag<T> bfs[EARLY ? 4 : 1][KS];
        if constexpr (EARLY) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) bfs[st][ks] = load_frag(ktile + (16 * st + n16) * ROW + 32 * ks + 8 * g);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 acc[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) acc[ht] = f4zero();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<T> bf;
                if constexpr (EARLY) bf = bfs[st][ks];
                else bf = load_frag(ktile + (16 * st + n16) * ROW + 32 * ks + 8 * g);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16(qa[ht][ks], bf, acc[ht]);
            }
            float v = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int i = 0; i < 4; ++i)      // ReLU on the bit pattern: negative floats are negative ints
                    v += wv[ht][i] * __int_as_float(max(__float_as_int(acc[ht][i]), 0));
            v = rows_sum(v);
            if (g == st) my = v;
        }
        my = my + 0.0f;                        // -0 -> +0: one value per tie class
        const int j = j0 + lane;
        const bool valid = j < nv && (!dcol || dcur == dt);
        const int ntile = min(KT, nv - j0);
        if (cnt + ntile > cap) {
            // make room: the loose cut when its bin allows, else the exact one
            const float hi = wave_max(rhi);
            int kept = 0;
            if constexpr (ROOM) {
                if (try_room) kept = select_room<SB>(bufs, cnt, kp, room_limit, wave_min(rlo), hi, tau);
            }
            if (kept > 0) {
                cnt = kept;
            } else {
                tau = select_keep<SB>(bufs, cnt, kp);
                cnt = kp;
            }
            rlo = tau;                                // the kept entries span [tau, hi]
            rhi = hi;
        }
        const bool take = valid && my > tau;
        const uint64_t m = __ballot(take);
        if (take) {
            const int p = cnt + (int)mbcnt(m);
            bufs.s[p] = my;
            bufs.j[p] = j;
            if constexpr (ROOM) {
                rlo = fminf(rlo, my);
                rhi = fmaxf(rhi, my);
            }
        }
        cnt += __popcll(m);
    }
    if (!active) return;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int kk = min(kp, nv);
    if (cnt > kk) {
        select_keep<SB>(bufs, cnt, kk);
        cnt = kk;
    }
    int32_t* orow = idx + row * kp;
    float* srow = score ? score + row * kp : nullptr;
    for (int i = lane; i < kp; i += WAVE) {
        const bool have = i < cnt;
        orow[i] = have ? bufs.j[i] : -1;
        if (srow) srow[i] = have ? bufs.s[i] : -INFINITY;
    }
}

template <typename T, int DI, int HT>
hipError_t launch_index(const IndexArgs& p, hipStream_t st)
{
    const int kp = p.kp;
    const int cap = index_topk_cap(p, sizeof(T) == 2);
    if (cap == 0) return hipErrorInvalidValue;
    const size_t lds = topk_lds_bytes(p.DI, sizeof(T), cap);
    auto kern = index_topk_kernel<T, DI, HT>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid((p.S + 3) / 4, p.b);
    TimedLaunch tl(K_INDEX_TOPK, st);
    const IndexStrides is{p.qsb, p.qss, p.qsh, p.ksb, p.kss, p.wsb, p.wss};
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, (const T*)p.qi, (const T*)p.ki, p.w, p.doc, p.idx,
                       p.score, p.S, p.HI, p.r, p.nc, kp, cap, is);
    return hipGetLastError();
}

template <typename T, int DI>
hipError_t launch_index_ht(const IndexArgs& p, hipStream_t st)
{
    if (p.HI <= 16) return launch_index<T, DI, 1>(p, st);
    return launch_index<T, DI, 4>(p, st);
}

}  // namespace

hipError_t index_topk(const IndexArgs& p, bool bf16, hipStream_t st)
{
    if (p.kp == 0 || p.S == 0) return hipSuccess;
    switch (p.DI) {
    case 32: return bf16 ? launch_index_ht<bf16_t, 32>(p, st) : launch_index_ht<float, 32>(p, st);
    case 64: return bf16 ? launch_index_ht<bf16_t, 64>(p, st) : launch_index_ht<float, 64>(p, st);
    case 128: return bf16 ? launch_index_ht<bf16_t, 128>(p, st) : launch_index_ht<float, 128>(p, st);
    default: return hipErrorInvalidValue;
    }
}

// Candidate-buffer capacity per query (entries): the whole valid prefix when
// it fits on chip (no cut ever happens), else twice K' rounded up to a tile,
// which leaves room for a full tile after every cut; the smaller size also
// when it lets two workgroups share a CU and the whole prefix does not (the
// cuts cost less than the lost occupancy).  0 = does not fit.
int index_topk_cap(const IndexArgs& p, bool bf16)
{
    const int elem = bf16 ? 2 : 4;
    const int nc64 = (p.nc + 63) / 64 * 64, kp64 = (p.kp + 63) / 64 * 64;
    int cap = nc64;
    const int small = 2 * kp64;
    const size_t lim = INDEX_LDS_LIMIT;
    if (small < cap && (topk_lds_bytes(p.DI, elem, cap) > lim ||
                        (2 * topk_lds_bytes(p.DI, elem, small) <= lim && 2 * topk_lds_bytes(p.DI, elem, cap) > lim)))
        cap = small;
    if (topk_lds_bytes(p.DI, elem, cap) > (size_t)INDEX_LDS_LIMIT) return 0;
    return cap;
}

}  // namespace csa
