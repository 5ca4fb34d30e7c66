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
// shared by its heads and the natural matrix-core tile is (heads x rows x d).
//
// Forward and dQ (query-major, sparse): the G waves of a query each own 16*HT
// of its heads and walk its candidate list in chunks of 32 rows (window rows
// first, then compressed slots).  The lanes gather a chunk's rows into
// registers while the previous chunk computes and store them into a
// double-buffered, swizzled LDS tile that the query's waves share; the
// logits read the tile as MFMA operands, and the contraction over rows reads
// it transposed with ds_read_b64_tr_b16.
//
// Variants of the same kernels: packed documents (an LDS bit per window or
// dense slot of the query's document); no window (W = 0: only selected rows;
// a query without a candidate gets O = 0 and LSE = -inf); rows packed as
// [k | v] with q = [q | 0] and dO = [0 | dO] (KSP > 0: the zero halves'
// products are skipped), which is how the grouped-query path runs through
// here; and in the key-stationary kernel, QS > 1 consecutive queries of few
// heads each stacked in the 64 head slots.
//
// dKV / dC (key-stationary, masked): fp32 atomics cannot absorb one add per
// (query, row, d) -- a row is selected by hundreds of queries -- so the row
// gradients are reduced on chip instead.  A workgroup owns a tile of key
// rows (kept in registers as MFMA operands) and a block of consecutive
// queries; it stages each query's q and dO in LDS and accumulates
// P^T dO + dS'^T q over the query block in registers, masking (query, row)
// pairs that are not candidates.  Partial sums per query block go to a
// workspace and one reduction kernel adds them up: no atomics, and the sum
// order is fixed.
#include <algorithm>
#include <array>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <type_traits>
#include <utility>
#include <vector>

#include "csa_device.hpp"
#include "csa_kernels.hpp"
#include "timing.hpp"

namespace csa {

namespace {

constexpr int CHUNK = 32;

template <typename T> constexpr int row_pad() { return 16 / (int)sizeof(T); }

// Candidate list of one query: window slots [0, nwin), then compressed slots.
template <typename T>
struct Cand {
    const T* kv;          // batch base of kv
    const T* c;           // batch base of c (nullptr: window only)
    const int32_t* irow;  // index row of the query (nullptr: dense mode)
    const uint32_t* okb;  // packed documents: LDS bit per window / dense slot, 1 = same document
    int64_t kst;          // element stride between consecutive kv rows
    int t, D, u0, nwin, nv, nslots;

    __device__ __forceinline__ void init(const AttnArgs& p, int bi, int tq)
    {
        t = tq;
        D = p.D;
        kv = (const T*)p.kv + (int64_t)bi * p.kvsb;
        kst = p.kvst;
        c = p.c ? (const T*)p.c + (int64_t)bi * p.nc * p.D : nullptr;
        irow = (p.c && p.idx) ? p.idx + ((int64_t)bi * p.S + tq) * p.kp : nullptr;
        okb = nullptr;
        nwin = min(p.W, tq + 1);
        u0 = tq - nwin + 1;
        nv = p.c ? min((tq + 1) / p.r, p.nc) : 0;
        const int ncs = p.c ? (p.idx ? p.kp : nv) : 0;
        nslots = nwin + ncs;
    }
    // Row code of a slot: u (window row), j | 0x40000000 (compressed row),
    // or -1 (invalid: padding, out of range, not yet valid, or another
    // document).  The index row is read from its copy `ids` in LDS.  Entries
    // of a given index row get no document test (the indexer already applied
    // it); window slots and dense-mode slots do.
    __device__ __forceinline__ bool ok_bit(int slot) const
    {
        return !okb || ((((const lds_u32*)okb)[slot >> 5] >> (slot & 31)) & 1u);
    }
    __device__ __forceinline__ int code(int slot, const int32_t* ids) const
    {
        if (slot < nwin) return ok_bit(slot) ? u0 + slot : -1;
        if (slot >= nslots) return -1;
        const int s2 = slot - nwin;
        const int j = irow ? ((const lds_i32*)ids)[s2] : s2;
        const bool ok = j >= 0 && j < nv && (irow || ok_bit(slot));
        return ok ? (j | 0x40000000) : -1;
    }
    __device__ __forceinline__ const T* row_ptr(int code) const
    {
        const bool isc = code >= 0 && (code & 0x40000000);
        const int row = code < 0 ? t : (code & 0x3fffffff);
        return isc ? c + (int64_t)row * D : kv + (int64_t)row * kst;
    }
};

// ------------------------------------------- forward / dQ (query-major)
// The G waves of a query (G = 1 unless head groups are split) share one
// double-buffered LDS tile per query.  Chunk k+1's rows are gathered from
// global memory into registers (each lane loads 16-byte pieces of its rows)
// while chunk k computes, and written to the other buffer afterwards; rows
// are stored with 8-element units permuted per row (unit u of row r at
// u ^ unit_swz(r)) so both reads below are free of bank conflicts.
// S^T[r, h] = R[r, :] . Q[h, :]      A = rows from LDS (m = r, k = d)
//                                    B = Q^T (k = d, n = h), registers
// forward: online softmax per column h (lane), base-2 exponentials, then
//   O^T[d, h] += R^T P^T              A = R^T through the transposing read,
//                                     B = P^T straight from the S^T accumulators
// dQ mode: dP^T = R . dO^T, scale*P^T = exp(S^T scale - lse), dS'^T = scale P^T (dP^T - Delta),
//   dQ^T[d, h] += R^T dS'^T           same operand shapes
template <typename T, int D> constexpr int chunk_bytes() { return CHUNK * D * (int)sizeof(T); }
// 32-row chunks a query's waves gather per round: two for the bf16 d <= 128
// forward whose heads take two waves (half the rounds, barriers and slot
// lookups per query; the tile pair still leaves room for four workgroups
// per CU), one elsewhere (the dq kernel has no registers for the larger
// gather).  The chunks of a round are processed in order.
template <typename T, int D, int G, bool DQ> constexpr int round_chunks()
{
    return (sizeof(T) == 2 && D <= 128 && G == 2 && !DQ) ? 2 : 1;
}
template <typename T, int D, int G, bool DQ> constexpr int round_bytes()
{
    return round_chunks<T, D, G, DQ>() * chunk_bytes<T, D>();
}

template <typename T, int D, int HT, int G, bool DQ, int KSP>
__global__ __launch_bounds__(256, (D <= 128 && HT <= 2) ? 2 : 1)
void attn_query_kernel(AttnArgs p, float* __restrict__ delta, float* __restrict__ csink, int idx_lds, int okw)
{
    constexpr int KS = D / 32, DT = D / 16, QPW = (G == 2 && D <= 128) ? 1 : 4 / G;
    constexpr int NSUB = round_chunks<T, D, G, DQ>();   // chunks per round
    constexpr int RR = NSUB * CHUNK;              // rows per round
    constexpr int CHB = round_bytes<T, D, G, DQ>();     // one round's tile
    constexpr int PPR = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
    constexpr int E16 = 16 / (int)sizeof(T);      // elements per piece
    constexpr int NPL = CHB / (16 * WAVE * G);    // pieces each lane of the query's waves carries
    static_assert(NPL * 16 * WAVE * G == CHB, "round pieces split evenly over the query's waves");
    static_assert(RR <= WAVE, "one lane resolves each slot of a round");
    typedef std::conditional_t<(RR > 32), uint64_t, uint32_t> mask_t;   // bit i: slot i of a round
    constexpr int LPR = WAVE * G / RR;            // lanes sharing one row of a round
    static_assert(LPR * NPL == PPR, "a row's pieces split evenly over its lanes");
    typedef uint32_t piece_t __attribute__((ext_vector_type(4)));
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int g = lane / 16, n16 = lane % 16;
    const int qs = wave / G, sub = wave % G;      // query slot in the workgroup, wave within the query
    char* tiles = smem + (size_t)qs * 2 * CHB;

    const int bi = blockIdx.y;
    // latest queries (longest candidate lists) first: short ones fill the tail
    const int t = ((int)gridDim.x - 1 - (int)blockIdx.x) * QPW + qs;
    const bool active = t < p.S;                  // inactive waves still join the barriers (G > 1)
    const int h0 = sub * 16 * HT;
    Cand<T> cand;
    cand.init(p, bi, active ? t : p.S - 1);
    const int64_t qrow = (int64_t)bi * p.S + (active ? t : p.S - 1);
    const int64_t qoff = (int64_t)bi * p.qsb + (int64_t)(active ? t : p.S - 1) * p.qst;   // q-like tensors
    const int64_t loff = (int64_t)bi * p.lsb + (int64_t)(active ? t : p.S - 1) * p.lst;   // lse
    const float sl2 = p.scale * LOG2E;
    [[maybe_unused]] const float isl2 = 1.f / sl2;
    [[maybe_unused]] const float lsc = __log2f(p.scale);
    const T* qp = (const T*)p.q + qoff;
    // The query's index row goes to LDS once (per-chunk slot lookups then do
    // not wait on memory).  Its loads are issued first, into registers, so
    // that they overlap the loads of Q (dO, O) below.
    int32_t* ids = reinterpret_cast<int32_t*>(smem + (size_t)QPW * 2 * CHB) + (size_t)qs * p.kp;
    const bool use_ids = cand.irow != nullptr;    // the host guarantees the LDS copy (idx_lds)
    constexpr int IPL = 2048 / (WAVE * G);        // index entries per lane, K' <= 2048
    const int qlane = sub * WAVE + lane;
    int iv[IPL];
    if (use_ids) {
#pragma unroll
        for (int k = 0; k < IPL; ++k) {
            const int s0 = qlane + k * WAVE * G;
            iv[k] = s0 < p.kp ? cand.irow[s0] : -1;
        }
    }

    // Packed documents: one LDS bit per window slot and (dense mode) per
    // compressed slot, set when the row's document is the query's (okw words
    // per query slot of the workgroup, after the index rows).
    if (okw > 0) {
        uint32_t* okq = reinterpret_cast<uint32_t*>(smem + (size_t)QPW * 2 * CHB +
                                                    (idx_lds ? (size_t)QPW * p.kp * sizeof(int32_t) : 0)) +
                        (size_t)qs * okw;
        const int32_t* dcol = p.doc + (int64_t)bi * p.S;
        const int dt = dcol[cand.t];
        const int nbits = cand.nwin + (cand.irow || !p.c ? 0 : cand.nv);
        for (int s0 = sub * WAVE; s0 < nbits; s0 += WAVE * G) {
            const int sl = s0 + lane;
            bool ok = false;
            if (sl < nbits) ok = dcol[sl < cand.nwin ? cand.u0 + sl : (sl - cand.nwin) * p.r] == dt;
            const uint64_t m = __ballot(ok);
            if (lane == 0) {
                okq[s0 >> 5] = (uint32_t)m;
                okq[(s0 >> 5) + 1] = (uint32_t)(m >> 32);
            }
        }
        cand.okb = okq;
    }

    Frag<T> qb[HT][KS];
    [[maybe_unused]] Frag<T> db[HT][KS];
    float m2[HT];
    [[maybe_unused]] f32x4 lsum[HT];              // softmax denominators (every element holds the head's)
    [[maybe_unused]] float lse2[HT], dlt[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + 16 * ht + n16;
        const bool hv = h < p.H;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ht][ks] = hv ? load_frag(qp + h * p.qsh + 32 * ks + 8 * g) : zero_frag<T>();
        if constexpr (!DQ) {
            // the running reference starts finite: a chunk whose rows are all
            // masked (another document) has logits -inf, and -inf against a
            // reference of -inf gives NaN; the sink's mass relative to the
            // reference seeds the sum
            const bool sk = p.sink && hv;
            const float sl = sk ? p.sink[h] * LOG2E : -INFINITY;
            m2[ht] = fmaxf(sl, -1e30f);
            const float l0 = sk ? fast_exp2(sl - m2[ht]) : 0.f;
            lsum[ht] = f32x4{l0, l0, l0, l0};
        } else {
            // Delta[h] = <dO[t, h], O[t, h]>; dO kept as the B operand of dP^T
            const T* dop = (const T*)p.dout + qoff + h * p.qsh;
            const T* op = (const T*)p.out + qoff + h * p.qsh;
            float part = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                db[ht][ks] = hv ? load_frag(dop + 32 * ks + 8 * g) : zero_frag<T>();
                if (hv) {
                    const Frag<T> of = load_frag(op + 32 * ks + 8 * g);
#pragma unroll
                    for (int e = 0; e < 8; ++e) part += to_f32(db[ht][ks].v[e]) * to_f32(of.v[e]);
                }
            }
            part = rows_sum(part);
            dlt[ht] = part;
            lse2[ht] = hv ? p.lse[loff + h] * LOG2E : INFINITY;
            if (active && hv && g == 0) {
                delta[qrow * p.H + h] = part;
                // this query's term of dsink[h], head-major; summed in a fixed order later
                if (csink) csink[(int64_t)h * p.b * p.S + qrow] = -fast_exp2(p.sink[h] * LOG2E - lse2[ht]) * part;
            }
        }
    }
    if constexpr (DQ) {
        if (!p.dq) return;                        // uniform over the workgroup
    }
    [[maybe_unused]] Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones.v[e] = (T)1.0f;
    // wide rows (d >= 256): the dQ accumulators live in AGPRs (inline-asm
    // MFMAs, read once after a drain), which frees the VGPRs the d = 512 dq
    // kernel otherwise spills; at d <= 128 the compiler's own allocation wins
    constexpr bool OACC = DQ && sizeof(T) == 2 && D >= 256 && (DT * HT == 16 || DT * HT == 32);
    // bf16 reads a chunk's transposed rows all at once (fp32, and the one-wave
    // 32-head dQ kernel, have no registers to spare for that)
    constexpr bool EARLY = sizeof(T) == 2 && !(DQ && G == 1 && HT == 2);
    // chunks gathered ahead into registers: two (the gather latency then
    // spans two rounds) where the registers allow it (the bf16 forward at
    // d <= 128 with heads split over waves, both bf16 kernels at d = 512 with
    // four waves per query); one elsewhere
    constexpr int GDEPTH = NSUB == 1 && ((!DQ && sizeof(T) == 2 && D <= 128 && !(G == 1 && HT == 2)) ||
                                         (sizeof(T) == 2 && D == 512 && G == 4)) ? 2 : 1;
    f32x4 o[DT][HT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o[dt][ht] = OACC ? agpr_zero() : f4zero();

    // Gather the rows of the round starting at slot c0 into registers; returns
    // the round's candidate mask (bit i: slot c0 + i).  Lane q = 64 sub + lane
    // of the query's waves owns row q / LPR of the round and its pieces
    // (q % LPR) + LPR k, k < NPL: it resolves that row's address itself, and
    // its loads differ by immediate offsets only.
    const int my_r = (sub * WAVE + lane) / LPR, my_j = (sub * WAVE + lane) % LPR;
    piece_t rg[GDEPTH][NPL];
    auto fetch = [&](int c0, piece_t (&r)[NPL]) -> mask_t {
        // lane l resolves slot c0 + l % RR; the lanes that load row my_r take
        // its code from lane my_r
        const int cl = cand.code(c0 + (lane & (RR - 1)), ids);
        const mask_t mask = (mask_t)__ballot(cl >= 0);
        const T* rp = cand.row_ptr(__shfl(cl, my_r)) + my_j * E16;
#pragma unroll
        for (int k = 0; k < NPL; ++k) r[k] = *reinterpret_cast<const piece_t*>(rp + k * LPR * E16);
        return mask;
    };
    // write the gathered rows to buffer buf, units permuted per row
    auto stash = [&](int buf, const piece_t (&r)[NPL]) {
        T* dst = reinterpret_cast<T*>(tiles + (size_t)buf * CHB) + my_r * D;
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int pos = (my_j + LPR * k) * E16;
            *reinterpret_cast<piece_t*>(dst + ((((pos >> 3) ^ unit_swz(my_r, D / 8))) << 3) + (pos & 7)) = r[k];
        }
    };

    auto process = [&](const T* tile, uint32_t mask) {
        // S^T (and dP^T) for every head tile first: straight-line MFMA work
        f32x4 s[HT][2];
        [[maybe_unused]] f32x4 dp[HT][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            // KSP > 0: rows packed as [k | v] (the first KSP k-steps are the key
            // half) with q = [q | 0] and dO = [0 | dO]: the logits read the key
            // half, dP the value half (the zero halves are skipped)
            Frag<T> ra[KS];
            const int r = 16 * rt + n16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (KSP > 0 && !DQ && ks >= KSP) ra[ks] = zero_frag<T>();
                else ra[ks] = load_frag(tile + r * D + (((4 * ks + g) ^ unit_swz(r, D / 8)) << 3));
            }
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                f32x4 acc = f4zero();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    if (KSP == 0 || ks < KSP) acc = mfma16(ra[ks], qb[ht][ks], acc);
                s[ht][rt] = acc;
                if constexpr (DQ) {
                    f32x4 a2 = f32x4{-dlt[ht], -dlt[ht], -dlt[ht], -dlt[ht]};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        if (KSP == 0 || ks >= KSP) a2 = mfma16(ra[ks], db[ht][ks], a2);
                    dp[ht][rt] = a2;
                }
            }
        }
        if (mask != 0xffffffffu) {              // partial chunk (rare): non-candidates get -inf
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((mask >> (16 * rt + 4 * g + i)) & 1u)) {
#pragma unroll
                        for (int ht = 0; ht < HT; ++ht) s[ht][rt][i] = -INFINITY;
                    }
        }
        Frag<T> pb[HT];
        if constexpr (!DQ) {
            // exponentials are taken against a reference m2 that moves only when
            // some logit of the wave exceeds it by more than 2^8 (then every
            // head re-bases); P <= 2^8 otherwise, and O / l is unchanged.  The
            // test needs only each lane's own maximum; the per-head maximum
            // (a cross-lane reduction) is formed on the rare re-base.
            bool need = false;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float thr = fmaf(m2[ht] + 8.f, isl2, 0.f);   // scale > 0: compare logits directly
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) need |= s[ht][rt][i] > thr;
            }
            if (__any(need)) {                     // rare
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    const float mloc = fmaxf(fmaxf(fmaxf(s[ht][0][0], s[ht][0][1]), fmaxf(s[ht][0][2], s[ht][0][3])),
                                             fmaxf(fmaxf(s[ht][1][0], s[ht][1][1]), fmaxf(s[ht][1][2], s[ht][1][3])));
                    const float m = rows_max(mloc);
                    const float mnew = fmaxf(m2[ht], m * sl2);
                    const float alpha = fast_exp2(m2[ht] - mnew);
                    lsum[ht] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[dt][ht] *= alpha;
                    m2[ht] = mnew;
                }
            }
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float negm = -m2[ht];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pb[ht].v[4 * rt + i] = from_f32<T>(fast_exp2(fmaf(s[ht][rt][i], sl2, negm)));
                // row sums on the matrix core: a ones row against P^T sums the
                // chunk's (rounded) P of head n in every row of the result
                lsum[ht] = mfma16(ones, pb[ht], lsum[ht]);
            }
        } else {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                // scale * P in one exponential: 2^(s*scale*log2e + log2(scale) - lse*log2e);
                // dp started at -Delta, so dp = dP - Delta
                const float off = lsc - lse2[ht];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ps = fast_exp2(fmaf(s[ht][rt][i], sl2, off));
                        pb[ht].v[4 * rt + i] = from_f32<T>(dp[ht][rt][i] * ps);
                    }
            }
        }
        // O^T += R^T P^T   (or dQ^T += R^T dS'^T); packed rows: O needs the
        // value half only, dQ the key half only
        if constexpr (OACC) {
            // AGPR accumulators: four d tiles per asm block (HT == 1, so
            // o[dt .. dt+3][0] are consecutive); 2 * KSP is a multiple of 4
            static_assert(HT == 1 && DT % 4 == 0 && (KSP == 0 || (2 * KSP) % 4 == 0), "OACC layout");
#pragma unroll
            for (int dt = 0; dt < DT; dt += 4) {
                if (KSP > 0 && (DQ ? dt >= 2 * KSP : dt < 2 * KSP)) continue;
                Frag<T> a[4], b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a[j] = rows_operand<T>(tile, D, 0, 16 * (dt + j), true);
                    b[j] = pb[0];
                }
                mfma16_4_acc(&o[dt][0], a, b);
            }
        } else if constexpr (EARLY) {
            // every transposing read is issued before the first MFMA (one LDS
            // round trip per chunk rather than one per d tile)
            Frag<T> rt[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                if (!(KSP > 0 && (DQ ? dt >= 2 * KSP : dt < 2 * KSP))) rt[dt] = rows_operand<T>(tile, D, 0, 16 * dt, true);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (KSP > 0 && (DQ ? dt >= 2 * KSP : dt < 2 * KSP)) continue;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) o[dt][ht] = mfma16(rt[dt], pb[ht], o[dt][ht]);
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (KSP > 0 && (DQ ? dt >= 2 * KSP : dt < 2 * KSP)) continue;
                const Frag<T> a = rows_operand<T>(tile, D, 0, 16 * dt, true);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) o[dt][ht] = mfma16(a, pb[ht], o[dt][ht]);
            }
        }
    };

    // Slots past the last candidate need no chunk (index rows usually end in
    // -1 padding).  The last valid index slot comes from the entries each lane
    // loaded, which it also writes to LDS.
    int lastc = -1;                               // last valid compressed slot (index into the row)
    if (use_ids) {
#pragma unroll
        for (int k = 0; k < IPL; ++k) {
            const int s0 = qlane + k * WAVE * G;
            if (s0 < p.kp) {
                ids[s0] = iv[k];
                if (iv[k] >= 0 && iv[k] < cand.nv) lastc = max(lastc, s0);
            }
        }
    } else {
        lastc = cand.nslots - cand.nwin - 1;      // dense mode: every valid block; window only: none
    }
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) lastc = max(lastc, __shfl_xor(lastc, o2));
    int last = active ? max(cand.nwin - 1, lastc >= 0 ? cand.nwin + lastc : -1) : -1;
    int nloop;
    if constexpr (G > 1) {
        // one barrier: the index row is in LDS, and every wave sees every
        // query's last slot; all waves of the workgroup run the same number of
        // barrier rounds, for the longest candidate list among its queries.
        // The slots borrow the second tile of query slot 0, first written
        // after the barrier that ends the prologue below.
        int* last_s = reinterpret_cast<int*>(smem + CHB);
        if (lane == 0) last_s[wave] = last;
        __syncthreads();
        nloop = 0;
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            int lq = -1;
#pragma unroll
            for (int w = 0; w < G; ++w) lq = max(lq, last_s[q * G + w]);
            if (q == qs) last = lq;
            nloop = max(nloop, (lq + RR) / RR);
        }
    }
    const int nch = (last + RR) / RR;             // rounds
    if constexpr (G == 1) nloop = nch;
    // every load so far (Q, dO, O, the index row) has landed: the loop below
    // then waits only on its own row gathers
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0)
    // Round k computes the rows of round k from one LDS tile, writes those of
    // round k+1 into the other and gathers round k + 1 + GDEPTH into
    // registers.  G > 1: round k+1 fully written, round k read by every wave,
    // before the next round reads k+1 and refills k's tile.  G == 1: a wave's
    // LDS accesses run in order, so its own reads of a tile finish before its
    // later writes to it.
    mask_t mk[3] = {0u, 0u, 0u};                  // masks of rounds k, k+1, k+2
    if (nch > 0) { mk[0] = fetch(0, rg[0]); stash(0, rg[0]); }
#pragma unroll
    for (int j = 1; j <= GDEPTH; ++j)
        if (nch > j) mk[j] = fetch(RR * j, rg[j % GDEPTH]);
    if constexpr (G > 1) __syncthreads();
    // r: the registers holding round k+1, which then receive round k + 1 + GDEPTH
    auto round = [&](int k, piece_t (&r)[NPL]) {
        if constexpr (NSUB == 1) {
            if (G == 1 || k < nch) process(reinterpret_cast<const T*>(tiles + (size_t)(k & 1) * CHB), mk[0]);
        } else if (k < nch) {
            const T* tile = reinterpret_cast<const T*>(tiles + (size_t)(k & 1) * CHB);
#pragma unroll
            for (int h = 0; h < NSUB; ++h) {
                // a chunk with no candidate (past the last one) adds nothing
                const uint32_t mh = (uint32_t)(mk[0] >> (CHUNK * h));
                if (mh != 0u) process(tile + h * CHUNK * D, mh);
            }
        }
        if (k + 1 < nch) {
            stash((k + 1) & 1, r);
            mk[0] = mk[1];
            mk[1] = mk[2];
        }
        if (k + 1 + GDEPTH < nch) mk[GDEPTH] = fetch(RR * (k + 1 + GDEPTH), r);
        if constexpr (G > 1) __syncthreads();
    };
    if constexpr (GDEPTH == 1) {
        for (int k = 0; k < nloop; ++k) round(k, rg[0]);
    } else {
        for (int k = 0; k < nloop; k += 2) {      // the register sets alternate
            round(k, rg[1]);
            if (k + 1 < nloop) round(k + 1, rg[0]);
        }
    }
    if constexpr (OACC) agpr_drain<DT * HT>(&o[0][0]);
    if (!active) return;
    // epilogue: lane holds X^T[d = 16 dt + 4g + i][h = h0 + 16 ht + n16]
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + 16 * ht + n16;
        if (h >= p.H) continue;
        if constexpr (!DQ) {
            // no candidate and no sink (possible without a window): O = 0, LSE = -inf
            const float lt = lsum[ht][0];
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            T* orow = (T*)p.out + qoff + h * p.qsh;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * g + i] = from_f32<T>(o[dt][ht][i] * inv);
            if (g == 0) p.lse[loff + h] = lt > 0.f ? (m2[ht] + log2f(lt)) * LN2 : -INFINITY;
        } else {
            T* drow = (T*)p.dq + qoff + h * p.qsh;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) drow[16 * dt + 4 * g + i] = from_f32<T>(o[dt][ht][i]);
        }
    }
}

// ------------------------------------ dKV / dC partials (key-stationary)
// Workgroup (tile slot x, query block y, batch z).  Tile slots [0, n_wt) are
// window tiles: rows u = t0 - W + 1 + i of the block's band, i in
// [x*TR, (x+1)*TR); the remaining slots are compressed tiles j in
// [x'*TR, (x'+1)*TR).  Wave w owns RW rows of the tile.
//   S[h, r]  = Q[h, :] . R[r, :]      A = Q from LDS (m = h), B = rows (regs)
//   dP[h, r] = dO[h, :] . R[r, :]
//   P = m(t, r) exp(scale S - lse), dS' = scale P (dP - Delta)   (m = multiplicity)
//   dR[r, d] += P^T dO + dS'^T Q      A = P^T / dS'^T from the S / dP
//                                     accumulators (lane (r, g) holds heads 4g+i
//                                     of head tiles 2kk, 2kk+1), B = dO / Q
//                                     from LDS through the transposing read
// Heads the key-stationary kernel stages per unit of its query loop: all 64
// of a query, or 32 (two units per query) when two stagings of 64 heads do
// not fit in LDS but two of 32 do (bf16 d = 512), so that the next unit
// always loads while this one computes.
template <typename T, int D> constexpr int rows_unit_heads()
{
    return 4 * 64 * D * (int)sizeof(T) + 8 * 1024 <= ATTN_LDS_LIMIT
               ? 64
               : (4 * 32 * D * (int)sizeof(T) + 8 * 1024 <= ATTN_LDS_LIMIT ? 32 : 64);
}
// q/dO staging buffers of the key-stationary kernel: two (the next unit
// loads while this one computes) when they fit in LDS, else one.
template <typename T, int D> constexpr int rows_stage_buffers()
{
    return 4 * rows_unit_heads<T, D>() * D * (int)sizeof(T) + 8 * 1024 <= ATTN_LDS_LIMIT ? 2 : 1;
}
// waves per workgroup and key rows per wave: a workgroup's tile is 256 rows at
// d <= 128 (64 at d = 512).  bf16 uses 8 waves of 32 rows: two waves per SIMD,
// so one wave's exponentials overlap the other's matrix work.
template <typename T, int D> constexpr int rows_waves_t() { return (sizeof(T) == 2 && D <= 128) ? 8 : 4; }
template <typename T, int D> constexpr int rows_per_wave_t() { return D <= 128 ? 256 / rows_waves_t<T, D>() : 16; }
// LDS bytes of the key-stationary kernel without / with its key-row tile
template <typename T, int D, int QS = 1> constexpr size_t rows_lds_base()
{
    return 2 * (size_t)rows_stage_buffers<T, D>() * rows_unit_heads<T, D>() * D * sizeof(T) + 4 * 64 * 4 +
           (size_t)3 * QS * rows_waves_t<T, D>() * rows_per_wave_t<T, D>() * 4;
}
template <typename T, int D> constexpr size_t rows_lds_tile()
{
    return (size_t)rows_waves_t<T, D>() * rows_per_wave_t<T, D>() * (D + 16 / sizeof(T)) * sizeof(T);
}
// LDS bytes of the next query's index row (one query per unit only; K' <= 2048)
template <int QS> constexpr size_t rows_lds_index() { return QS == 1 ? 2048 * sizeof(int32_t) : 0; }
// bf16 rows at d <= 128 stay in registers (64 VGPRs next to the AGPR
// accumulators): the tile would be re-read from LDS for every head tile.
template <typename T, int D> constexpr bool rows_tile_in_lds()
{
    return !(sizeof(T) == 2 && D <= 128) && rows_lds_base<T, D>() + rows_lds_tile<T, D>() <= (size_t)ATTN_LDS_LIMIT;
}

// Workgroup schedule of the key-stationary kernel: with nmap > 0 the grid
// has nmap workgroups and workgroup i takes unit map[i] = (batch, query
// block) index * tiles + tile slot (ROWS_IDLE: none); the host fills the
// table so that every unit of one query block runs on one XCD and the XCDs
// get equal work.  nmap = 0: the closed-form round-robin schedule.
constexpr int ROWS_MAP_MAX = 768;
constexpr uint16_t ROWS_IDLE = 0xffff;
struct RowsGeom {
    int Qb, nqb, WB, n_wt, n_ct, TR;   // query block, blocks, band rows, tiles, tile rows
    int64_t sink_off;                  // float offset of the per-query dsink terms [H, b*S]
    int64_t win_off, comp_off;         // float offsets of the two partial regions in the workspace
    int nmap;
    uint16_t map[ROWS_MAP_MAX];
};

template <typename T, int D, int RW, int NW, int QS, int KSP>
__global__ __launch_bounds__(64 * NW, 1) void attn_rows_kernel(AttnArgs p, RowsGeom geo,
                                                           const float* __restrict__ delta,
                                                           float* __restrict__ ws)
{
    constexpr int KS = D / 32, DT = D / 16, RT = RW / 16, TR = NW * RW, NT = 64 * NW;
    constexpr int HP = 64;                       // heads, padded to 4 head tiles
    // QS > 1 (key/value groups of few heads, no window): the 64 head slots
    // hold HS heads of each of QS consecutive queries, which share the tile's
    // rows; slot h belongs to query t + h / HS, head h % HS
    constexpr int HS = HP / QS;
    constexpr int CTR = QS * NW * RW;            // multiplicities per count buffer
    static_assert(QS == 1 || HS >= 4, "a lane's four head slots belong to one query");
    constexpr int HU = rows_unit_heads<T, D>();  // heads staged per unit of the query loop
    constexpr int NU = HP / HU;                  // units per query
    static_assert(HU == HP || QS == 1, "stacked queries stage all head slots at once");
    constexpr int QELEMS = HU * D;               // one staged q (or dO) block
    constexpr int NBUF = rows_stage_buffers<T, D>();
    constexpr int L16 = QELEMS * (int)sizeof(T) / 16;   // 16-byte pieces per block
    static_assert(L16 % NT == 0, "staging: whole 1 KiB wave loads");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // [buf 0: q, dO][buf 1: q, dO (double buffering only)][lse x2][Delta x2][mult x3]
    T* stage_base = reinterpret_cast<T*>(smem);
    float* lse_lds = reinterpret_cast<float*>(smem + 2 * NBUF * (size_t)QELEMS * sizeof(T));
    float* dlt_lds = lse_lds + 2 * HP;
    unsigned* cnt_lds = reinterpret_cast<unsigned*>(dlt_lds + 2 * HP);

    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int g = lane / 16, n16 = lane % 16;
    // Workgroups go to the 8 XCDs round-robin by linear id.  All tiles of one
    // query block are mapped to the same XCD, so its staged q / dO rows are
    // fetched from HBM once into that XCD's L2.  Without a schedule table,
    // query blocks are dealt to the XCDs in turn, heaviest (latest queries:
    // longest valid prefix) first; the table (rows_geometry) balances them.
    const int ntiles = geo.n_wt + (p.c ? geo.n_ct : 0);
    const int lin = blockIdx.x;
    int qbi, slot;                               // index over (batch, query block); tile slot
    if (geo.nmap > 0) {
        const int e = geo.map[lin];
        if (e == ROWS_IDLE) return;
        qbi = e / ntiles;
        slot = e % ntiles;
    } else {
        const int xcd = lin & 7, kx = lin >> 3;
        qbi = (kx / ntiles) * 8 + xcd;
        slot = kx % ntiles;
    }
    if (qbi >= p.b * geo.nqb) return;
    const int bi = qbi / geo.nqb, qb = geo.nqb - 1 - qbi % geo.nqb;
    const int t0 = qb * geo.Qb, t1 = min(p.S, t0 + geo.Qb);
    const bool win = slot < geo.n_wt;
    const int tile = win ? slot : slot - geo.n_wt;
    const int i0 = tile * TR;                    // first partial row of the tile
    int base_row, nrows_valid;                   // key row of partial row 0; rows that are meaningful
    if (win) {
        if (i0 >= geo.WB) return;
        base_row = t0 - p.W + 1;
        nrows_valid = geo.WB;
    } else {
        const int nvmax = min(t1 / p.r, p.nc);
        if (i0 >= nvmax) return;
        base_row = 0;
        nrows_valid = nvmax;
    }
    const T* rows = win ? (const T*)p.kv + (int64_t)bi * p.kvsb : (const T*)p.c + (int64_t)bi * p.nc * D;
    const int64_t rstride = win ? p.kvst : (int64_t)D;
    const int rmax = win ? p.S : p.nc;
    const int tile_lo = base_row + i0;           // key range of the tile
    const int tile_hi = base_row + min(i0 + TR, nrows_valid);
    // queries of the block that can reach the tile: a contiguous range
    int ta, tb;
    if (win) {
        ta = max(t0, tile_lo);
        tb = min(t1, tile_hi + p.W - 1);
    } else {
        ta = max(t0, (tile_lo + 1) * p.r - 1);
        tb = t1;
    }

    // this wave's rows as B operands (k = d, n = r): in registers, or (when the
    // LDS budget allows) in a wave-private LDS tile to leave registers for S / dP
    constexpr bool ROWS_LDS = rows_tile_in_lds<T, D>();
    constexpr int RROW = D + row_pad<T>();
    T* rtile = reinterpret_cast<T*>(reinterpret_cast<char*>(cnt_lds) + 3 * CTR * 4) + (size_t)wave * RW * RROW;
    Frag<T> rb[ROWS_LDS ? 1 : RT][KS];
    int rkey[RT];
    [[maybe_unused]] int rdoc[RT];               // packed documents: document of each window row
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int i = i0 + RW * wave + 16 * rt + n16;
        const int key = base_row + i;
        const bool ok = i < nrows_valid && key >= 0 && key < rmax;
        rkey[rt] = ok ? key : -1;
        rdoc[rt] = (p.doc && win && ok) ? p.doc[(int64_t)bi * p.S + key] : 0;
        const T* src = rows + (int64_t)(ok ? key : 0) * rstride;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const Frag<T> f = load_frag(src + 32 * ks + 8 * g);
            if constexpr (ROWS_LDS) store_frag(rtile + (16 * rt + n16) * RROW + 32 * ks + 8 * g, f);
            else rb[rt][ks] = f;
        }
    }
    f32x4 acc[RT][DT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = sizeof(T) == 2 ? agpr_zero() : f4zero();

    // Stage q[t] and dO[t] into buffer `buf` with asynchronous global->LDS
    // loads.  16-byte piece s of the block lands at LDS piece s; its source is
    // chosen so that the LDS block holds rows of 8-element units permuted as
    // unit u of row h at u ^ unit_swz(h).  Also lse, Delta (plain loads) and the
    // multiplicities of the tile's rows for query t in cnt buffer `cb`.
    // The next query's index row goes to LDS (after the other areas) with
    // asynchronous loads: entry s lands where thread s % NT reads it back in
    // count(), and no register waits on it while the unit computes.
    constexpr int IDX_REGS = 2048 / NT;           // K' <= 2048
    [[maybe_unused]] int32_t* const idx_buf = reinterpret_cast<int32_t*>(
        smem + rows_lds_base<T, D, QS>() + (rows_tile_in_lds<T, D>() ? rows_lds_tile<T, D>() : 0));
    // stacked queries with a selection bitmap: stage() loads the bitmap words
    // of the stack's (query, tile row) entries and the queries' repeat flags,
    // and the following count() turns them into multiplicities
    static_assert(QS == 1 || CTR % NT == 0, "whole bitmap entries per thread");
    constexpr int SEL_REGS = QS > 1 ? CTR / NT : 1;
    [[maybe_unused]] uint32_t sword[SEL_REGS];
    [[maybe_unused]] uint32_t srep = 0u;
    // hu: which HU heads of query t (unit hu of the query); the index row and
    // dense multiplicities are loaded with the query's first unit only
    float st_l = 0.f, st_d = 0.f;                 // LSE and Delta of the staged unit's head slot
    bool st_hv = false;
    auto stage = [&](int t, int hu, int buf, int cb) {
        const int64_t qrow = (int64_t)bi * p.S + t;
        const int64_t qoff = (int64_t)bi * p.qsb + (int64_t)t * p.qst;
        const T* qsrc = (const T*)p.q + qoff;
        const T* dsrc = (const T*)p.dout + qoff;
        T* qdst = stage_base + (size_t)(2 * buf) * QELEMS;
        T* ddst = qdst + QELEMS;
        constexpr int PER_ROW = D * (int)sizeof(T) / 16;   // 16-byte pieces per row
#pragma unroll
        for (int k = 0; k < L16 / NT; ++k) {
            const int piece = (k * NW + wave) * WAVE + lane;
            const int h = piece / PER_ROW, pr = piece % PER_ROW;
            // piece pr of LDS row h holds elements [pr*E, pr*E+E) of the permuted row
            constexpr int E = 16 / (int)sizeof(T);
            const int pos = pr * E;                       // element position in LDS row
            const int unit = (pos >> 3) ^ unit_swz(h, D / 8);   // source unit
            const int srcel = (unit << 3) | (pos & 7);
            const size_t wbase = (size_t)(k * NW + wave) * WAVE * 16;  // wave's 1 KiB in bytes
            const T* qp = qsrc;
            const T* dp_ = dsrc;
            if constexpr (QS == 1) {
                const int gh = hu * HU + h;
                const int hh = gh < p.H ? gh : 0;         // padded heads read row 0 (masked later)
                qp += hh * p.qsh + srcel;
                dp_ += hh * p.qsh + srcel;
            } else {
                // stacked slots: query t + h / HS, head h % HS (slots past the block read row 0 of t)
                const int tq = t + h / HS, hq = h % HS;
                const int64_t soff = (hq < p.H && tq < tb) ? (int64_t)(tq - t) * p.qst + (int64_t)hq * p.qsh : 0;
                qp += soff + srcel;
                dp_ += soff + srcel;
            }
            __builtin_amdgcn_global_load_lds((const void*)qp,
                                             (__attribute__((address_space(3))) void*)((char*)qdst + wbase), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)dp_,
                                             (__attribute__((address_space(3))) void*)((char*)ddst + wbase), 16, 0, 0);
        }
        if (threadIdx.x < HU) {
            // the LSE and Delta of head slot threadIdx.x, into registers only:
            // stage_params() writes them to LDS once they have landed (a wait
            // here would also wait for the staging loads just issued)
            if constexpr (QS == 1) {
                const int h = hu * HU + (int)threadIdx.x;
                st_hv = h < p.H;
                st_l = st_hv ? p.lse[(int64_t)bi * p.lsb + (int64_t)t * p.lst + h] : 0.f;
                st_d = st_hv ? delta[qrow * p.H + h] : 0.f;
            } else {
                const int h = threadIdx.x;
                const int tq = t + h / HS, hq = h % HS;
                st_hv = hq < p.H && tq < tb;
                const int64_t hrow = (qrow + (tq - t)) * p.H + hq;
                st_l = st_hv ? p.lse[(int64_t)bi * p.lsb + (int64_t)tq * p.lst + hq] : 0.f;
                st_d = st_hv ? delta[hrow] : 0.f;
            }
        }
        if (!win && QS == 1 && hu == 0) {
            if (p.idx) {
                // index entries are only loaded here; count() consumes them later
                const int32_t* irow = p.idx + qrow * p.kp;
#pragma unroll
                for (int k = 0; k < IDX_REGS; ++k) {
                    const int s = threadIdx.x + NT * k;
                    if (s < p.kp)
                        __builtin_amdgcn_global_load_lds((const void*)(irow + s),
                                                         (__attribute__((address_space(3))) void*)(idx_buf + NT * k +
                                                                                                   WAVE * wave),
                                                         4, 0, 0);
                }
            } else {
                unsigned* cnt = cnt_lds + cb * CTR;
                const int nv = min((t + 1) / p.r, p.nc);
                // dense mode: every valid block once (with documents: blocks of t's document)
                if (p.doc) {
                    const int32_t* dcol = p.doc + (int64_t)bi * p.S;
                    const int dt = dcol[t];
                    for (int j = tile_lo + threadIdx.x; j < min(tile_hi, nv); j += NT)
                        if (dcol[j * p.r] == dt) cnt[j - tile_lo] = 1u;
                    // settle these loads on their own path: a later wait for
                    // their registers would be a wait for every load, the
                    // staging included, on every path
                    __builtin_amdgcn_s_waitcnt(0x0F70);
                } else {
                    for (int j = tile_lo + threadIdx.x; j < min(tile_hi, nv); j += NT) cnt[j - tile_lo] = 1u;
                }
            }
        }
        if constexpr (QS > 1) {
            if (!win && p.idx && p.selmap) {
                const uint32_t* mrow = p.selmap + (int64_t)bi * p.S * p.selw;
#pragma unroll
                for (int k = 0; k < SEL_REGS; ++k) {
                    const int e = threadIdx.x + NT * k, tq = t + e / TR, key = tile_lo + e % TR;
                    sword[k] = (tq < tb && key < tile_hi) ? mrow[(int64_t)tq * p.selw + (key >> 5)] : 0u;
                }
                srep = (lane < QS && t + lane < tb) ? mrow[(int64_t)(t + lane) * p.selw + p.selw - 1] : 0u;
            }
        }
    };
    // initial values of the S and dP accumulators of each head slot of the
    // staged unit, into LDS buffer buf: the logit offset -lse/scale (so that
    // scale*log2e*S' = log2 P) and -Delta (a query with no candidate has
    // LSE = -inf and multiplicity 0 everywhere: any finite offset keeps its P
    // at 0)
    auto stage_params = [&](int buf) {
        if (threadIdx.x < HU) {
            lse_lds[buf * HP + threadIdx.x] = st_hv ? (st_l > -INFINITY ? -st_l / p.scale : 0.f) : -INFINITY;
            dlt_lds[buf * HP + threadIdx.x] = st_hv ? -st_d : 0.f;
        }
    };
    // multiplicities of the tile's rows for query t from the staged index entries
    auto count = [&](int t, int cb) {
        if (win || !p.idx) return;
        unsigned* cnt = cnt_lds + cb * CTR;
        if constexpr (QS > 1) {
            // bitmap path: every wave loaded the same repeat flags, so all
            // threads take the same branch; a bit is a multiplicity of 0 or 1
            if (p.selmap && !__any(srep != 0u)) {
#pragma unroll
                for (int k = 0; k < SEL_REGS; ++k) {
                    const int e = threadIdx.x + NT * k, key = tile_lo + e % TR;
                    cnt[e] = (sword[k] >> (key & 31)) & 1u;
                }
                return;
            }
            // a stack with a repeated entry (or no bitmap): its index rows, read here
            for (int qs = 0; qs < QS && t + qs < tb; ++qs) {
                const int tq = t + qs;
                const int nvq = min((tq + 1) / p.r, p.nc);
                const int32_t* irow = p.idx + ((int64_t)bi * p.S + tq) * p.kp;
                for (int s = threadIdx.x; s < p.kp; s += NT) {
                    const int j = irow[s];
                    if (j >= 0 && j < nvq && j >= tile_lo && j < tile_hi) atomicAdd(&cnt[qs * (NW * RW) + j - tile_lo], 1u);
                }
            }
            return;
        }
        const int nv = min((t + 1) / p.r, p.nc);
        __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this thread's index entries have landed
#pragma unroll
        for (int k = 0; k < IDX_REGS; ++k) {
            const int s = threadIdx.x + NT * k;
            const int j = s < p.kp ? idx_buf[s] : -1;
            if (j >= 0 && j < nv && j >= tile_lo && j < tile_hi) atomicAdd(&cnt[j - tile_lo], 1u);
        }
    };

    if (!win) {
        for (int i = threadIdx.x; i < 3 * CTR; i += NT) cnt_lds[i] = 0u;
        __syncthreads();
    }
    const float sl2 = p.scale * LOG2E;
    if (NBUF == 2 && ta < tb) {
        stage(ta, 0, 0, 0);
        stage_params(0);
        count(ta, 0);
    }
    // waves none of whose rows is a key of this tile only stage and synchronise
    // (their own loop copy: no branch around the accumulators inside the loop;
    // their partial rows are past the tile or at negative keys, never read)
    bool live = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) live |= rkey[rt] >= 0;
    live = __any(live);
    auto query_loop = [&](auto compute_tag) {
    constexpr bool COMPUTE = decltype(compute_tag)::value;
    // unit u: heads [HU hu, HU hu + HU) of query t = ta + QS (u / NU), hu = u % NU
    const int nunits = (tb - ta + QS - 1) / QS * NU;
    for (int u = 0; u < nunits; ++u) {
        const int it = u / NU, hu = u % NU;
        const int t = ta + it * QS;
        const int buf = NBUF == 2 ? (u & 1) : 0, cb = it % 3;
        if constexpr (NBUF == 2) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();                               // stage(u) visible; compute(u-1) done
            if (u + 1 < nunits) stage(ta + ((u + 1) / NU) * QS, (u + 1) % NU, buf ^ 1, ((u + 1) / NU) % 3);
        } else {
            __syncthreads();                               // compute(u-1) done with the buffer
            stage(t, hu, 0, cb);
            if (hu == 0) count(t, cb);
            __builtin_amdgcn_s_waitcnt(0);
            stage_params(0);
            __syncthreads();                               // stage(u) visible
        }
        if (!win && hu == 0) {                             // buffer of query it+2: last read by query it-1
            unsigned* nxt = cnt_lds + ((it + 2) % 3) * CTR;
            for (int i = threadIdx.x; i < CTR; i += NT) nxt[i] = 0u;
        }
        const T* q_lds = stage_base + (size_t)(2 * buf) * QELEMS;
        const T* do_lds = q_lds + QELEMS;
        const float* ls_b = lse_lds + buf * HP;
        const float* dl_b = dlt_lds + buf * HP;
        if constexpr (COMPUTE) {
        [[maybe_unused]] int dtq = 0;
        if (p.doc && win) {
            dtq = p.doc[(int64_t)bi * p.S + t];
            __builtin_amdgcn_s_waitcnt(0x0F70);    // settled on its own path, as in stage()
        }
        // every (head, row) pair of a wave with a candidate of t is computed;
        // its rows that are not candidates get multiplicity 0.  The
        // multiplicity enters the exponent: m P = 2^(scale log2e S' + log2 m).
        float lm[RT];                                      // log2 of the multiplicity, -inf for 0
        [[maybe_unused]] float lmq[QS > 1 ? 4 : 1][RT];   // stacked queries: per head tile
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int key = rkey[rt];
            float m = 0.f;
            if (key >= 0) {
                if (win) m = (key <= t && key > t - p.W && (!p.doc || rdoc[rt] == dtq)) ? 1.f : 0.f;
                else m = (float)cnt_lds[cb * CTR + key - tile_lo];
            }
            lm[rt] = m > 0.f ? __log2f(m) : -INFINITY;
            if constexpr (QS > 1) {
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                    const int qs = (16 * ht + 4 * g) / HS;     // this lane's query in the stack
                    const float mq = key >= 0 ? (float)cnt_lds[cb * CTR + qs * (NW * RW) + key - tile_lo] : 0.f;
                    lmq[ht][rt] = mq > 0.f ? __log2f(mq) : -INFINITY;
                }
            }
        }
        // a wave none of whose rows is a candidate of t (outside t's window,
        // not selected by t) skips t's products; it still stages and meets
        // the barriers with the others
        bool anyrow = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if constexpr (QS > 1) {
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) anyrow |= lmq[ht][rt] > -INFINITY;
            } else {
                anyrow |= lm[rt] > -INFINITY;
            }
        }
        if (__any(anyrow)) {
#pragma unroll
        for (int kk = 0; kk < HU / 32; ++kk) {
            // a head pair with no head (h <= 32); not in the bf16 d = 128
            // instantiation, where the branch costs more than it saves at h = 64
            if constexpr (!(sizeof(T) == 2 && D == 128) && QS == 1) {
                if (32 * (hu * (HU / 32) + kk) >= p.H) break;
            }
            Frag<T> pa[RT], sa[RT];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ht = 2 * kk + hh;
                f32x4 s0, d0;                              // accumulator starts: -lse/scale, -Delta
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s0[i] = ls_b[16 * ht + 4 * g + i];
                    d0[i] = dl_b[16 * ht + 4 * g + i];
                }
                Frag<T> qa[KS], da[KS];
                const int hrow = 16 * ht + n16;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = hrow * D + (((4 * ks + g) ^ unit_swz(hrow, D / 8)) << 3);   // d = 32 ks + 8 g
                    // packed [k | v] rows (KSP > 0): q lives in the key half, dO in the value half
                    qa[ks] = (KSP > 0 && ks >= KSP) ? zero_frag<T>() : load_frag(q_lds + off);
                    da[ks] = (KSP > 0 && ks < KSP) ? zero_frag<T>() : load_frag(do_lds + off);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    f32x4 sv = s0, dp = d0;
                    if constexpr (sizeof(T) == 2 && D == 128 && !ROWS_LDS && KSP == 0) {
                        mfma16_sd4_arows(sv, dp, qa, da, rb[rt]);
                    } else {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        Frag<T> bk;
                        if constexpr (ROWS_LDS) bk = load_frag(rtile + (16 * rt + n16) * RROW + 32 * ks + 8 * g);
                        else bk = rb[rt][ks];
                        if (KSP == 0 || ks < KSP) sv = mfma16(qa[ks], bk, sv);
                        if (KSP == 0 || ks >= KSP) dp = mfma16(da[ks], bk, dp);
                    }
                    }
                    // sv = S - lse/scale, dp = dP - Delta:  m P = 2^(sv sl2 + lm),
                    // scaled dS = scale (m P) (dP - Delta)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float lmv = lm[rt];
                        if constexpr (QS > 1) lmv = lmq[ht][rt];
                        const float e = fast_exp2(fmaf(sv[i], sl2, lmv));
                        pa[rt].v[4 * hh + i] = from_f32<T>(e);
                        sa[rt].v[4 * hh + i] = from_f32<T>((dp[i] * p.scale) * e);
                    }
                }
                // (no scheduling barrier here or between head-tile pairs: the S /
                // dP MFMAs of the next head tile interleave with this tile's
                // exponentials)
            }
            // dR += P^T dO + dS'^T q; bf16 accumulates in AGPRs through asm
            // blocks of 8 (or 4) MFMAs.  Packed rows: the key half of dR is
            // dS'^T q, the value half P^T dO (2 * KSP is a multiple of 4, so a
            // group of four d tiles lies in one half).
            if constexpr (sizeof(T) == 2 && RT == 2) {
                static_assert(KSP == 0 && DT % 2 == 0, "two-row-tile blocks");
                // the operands of the next two d-tile pairs are in flight while
                // a pair feeds the matrix cores (scheduling fences keep the
                // reads ahead of the products)
                Frag<T> dob[3][2], qbf[3][2];
                auto ld = [&](int dt, int b) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        dob[b][j] = rows_operand<T>(do_lds, D, 32 * kk, 16 * (dt + j), true);
                        qbf[b][j] = rows_operand<T>(q_lds, D, 32 * kk, 16 * (dt + j), true);
                    }
                };
                ld(0, 0);
                ld(2, 1);
#pragma unroll
                for (int dt = 0; dt < DT; dt += 2) {
                    const int b = (dt / 2) % 3;
                    if (dt + 4 < DT) ld(dt + 4, (dt / 2 + 2) % 3);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma16_2x2_acc(acc[0][dt], acc[0][dt + 1], acc[1][dt], acc[1][dt + 1], pa, sa, dob[b], qbf[b]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if constexpr (sizeof(T) == 2 && RT == 1) {
                static_assert(DT % 4 == 0 && (KSP == 0 || (2 * KSP) % 4 == 0), "one-row-tile blocks");
#pragma unroll
                for (int dt = 0; dt < DT; dt += 4) {
                    const bool khalf = KSP > 0 && dt < 2 * KSP, vhalf = KSP > 0 && dt >= 2 * KSP;
                    Frag<T> dob[4], qbf[4], pp[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        dob[j] = khalf ? zero_frag<T>() : rows_operand<T>(do_lds, D, 32 * kk, 16 * (dt + j), true);
                        qbf[j] = vhalf ? zero_frag<T>() : rows_operand<T>(q_lds, D, 32 * kk, 16 * (dt + j), true);
                        pp[j] = khalf ? sa[0] : pa[0];
                    }
                    if (khalf) mfma16_4_acc(&acc[0][dt], pp, qbf);
                    else if (vhalf) mfma16_4_acc(&acc[0][dt], pp, dob);
                    else mfma16_1x4_acc(&acc[0][dt], pa[0], sa[0], dob, qbf);
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bool khalf = KSP > 0 && dt < 2 * KSP, vhalf = KSP > 0 && dt >= 2 * KSP;
                    const Frag<T> dob = khalf ? zero_frag<T>() : rows_operand<T>(do_lds, D, 32 * kk, 16 * dt, true);
                    const Frag<T> qbf = vhalf ? zero_frag<T>() : rows_operand<T>(q_lds, D, 32 * kk, 16 * dt, true);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        if (!khalf) mfma16_acc(acc[rt][dt], pa[rt], dob);
                        if (!vhalf) mfma16_acc(acc[rt][dt], sa[rt], qbf);
                    }
                }
            }
        }
        }
        }
        if constexpr (NBUF == 2) {
            // the next unit's LSE / Delta and the next query's index loads
            // (issued with the staging) had compute(u) to land
            if (u + 1 < nunits) stage_params(buf ^ 1);
            if (hu == NU - 1 && t + QS < tb) count(t + QS, (it + 1) % 3);
        }
    }
    };
    if (!live) {                                           // no partial row of this wave is ever read
        query_loop(std::false_type{});
        return;
    }
    query_loop(std::true_type{});
    if constexpr (sizeof(T) == 2) agpr_drain<RT * DT>(&acc[0][0]);
    // partial rows of this wave: lane holds dR[r = 16 rt + 4g + i][d = 16 dt + n16]
    float* part = ws + (win ? geo.win_off + (((int64_t)bi * geo.nqb + qb) * geo.WB) * D
                            : geo.comp_off + (((int64_t)bi * geo.nqb + qb) * p.nc) * D);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pr = i0 + RW * wave + 16 * rt + 4 * g + i;
            if (pr >= nrows_valid) continue;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) part[(int64_t)pr * D + 16 * dt + n16] = acc[rt][dt][i];
        }
}

// dKV[b, u] = sum of the window partials of the query blocks whose band holds u;
// dC[b, j]  = sum of the compressed partials of the query blocks that reach j.
// One thread per (row, 4 consecutive d); the sum runs over query blocks in order.
// Blocks from `row_blocks` on: dsink[h] = sum over all queries of their terms
// (one block per head, a fixed summation order).
template <int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnArgs p, RowsGeom geo, const float* __restrict__ ws,
                                                          int row_blocks)
{
    constexpr int V = D / 4;
    if ((int)blockIdx.x >= row_blocks) {
        __shared__ float part[256];
        const int h = blockIdx.x - row_blocks;
        const int64_t n = (int64_t)p.b * p.S;
        const float* src = ws + geo.sink_off + (int64_t)h * n;
        float acc = 0.f;
        for (int64_t i = threadIdx.x; i < n; i += 256) acc += src[i];
        part[threadIdx.x] = acc;
        __syncthreads();
#pragma unroll
        for (int w = 128; w >= 1; w >>= 1) {
            if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) p.dsink[h] = part[0];
        return;
    }
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nkv = (int64_t)p.b * p.S * V;
    const int64_t nct = (int64_t)p.b * p.nc * V;
    if (tid < nkv) {
        const int v = tid % V;
        const int64_t row = tid / V;
        const int bi = (int)(row / p.S), u = (int)(row % p.S);
        const int q_lo = u / geo.Qb;
        const int q_hi = p.W > 0 ? min(geo.nqb - 1, (u + p.W - 1) / geo.Qb) : q_lo - 1;   // no window: zero
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
        for (int q = q_lo; q <= q_hi; ++q) {
            const int i = u - (q * geo.Qb - p.W + 1);
            const float4 x = *reinterpret_cast<const float4*>(
                ws + geo.win_off + (((int64_t)bi * geo.nqb + q) * geo.WB + i) * D + 4 * v);
            s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
        }
        *reinterpret_cast<float4*>(p.dkv + (int64_t)bi * p.kvsb + (int64_t)u * p.kvst + 4 * v) = s;
    } else if (tid < nkv + nct) {
        const int64_t k = tid - nkv;
        const int v = k % V;
        const int64_t row = k / V;
        const int bi = (int)(row / p.nc), j = (int)(row % p.nc);
        const int q_lo = ((j + 1) * p.r + geo.Qb - 1) / geo.Qb - 1;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
        for (int q = max(q_lo, 0); q < geo.nqb; ++q) {
            const float4 x = *reinterpret_cast<const float4*>(
                ws + geo.comp_off + (((int64_t)bi * geo.nqb + q) * p.nc + j) * D + 4 * v);
            s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
        }
        *reinterpret_cast<float4*>(p.dc + row * D + 4 * v) = s;
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

// ------------------------------------------------------------------ host
int rows_per_wave(int D) { return D <= 128 ? 64 : 16; }

namespace {

// Layout of the key-stationary kernel's units and workspace for query blocks
// of qb queries.
void rows_layout(RowsGeom& g, const AttnArgs& p, int qb)
{
    const int64_t D = p.D;
    g.TR = 4 * rows_per_wave(p.D);
    g.Qb = qb;
    g.nqb = (p.S + qb - 1) / qb;
    g.WB = p.W > 0 ? p.W - 1 + qb : 0;           // no window: no band rows
    g.n_wt = (g.WB + g.TR - 1) / g.TR;
    g.n_ct = p.nc > 0 ? (p.nc + g.TR - 1) / g.TR : 0;
    const int64_t delta_floats = ((int64_t)p.b * p.S * p.H + 63) / 64 * 64;
    g.sink_off = delta_floats;
    g.win_off = g.sink_off + delta_floats;
    g.comp_off = g.win_off + (int64_t)p.b * g.nqb * g.WB * D;
    g.nmap = 0;
}

int64_t rows_partial_floats(const AttnArgs& p, int qb)
{
    const int nqb = (p.S + qb - 1) / qb;
    return (int64_t)p.b * nqb * ((int64_t)(p.W > 0 ? p.W - 1 + qb : 0) + p.nc) * p.D;
}

// Queries that unit (query block qb, tile slot) walks, as the kernel derives
// them; -1 when the unit exits at once.
int rows_unit_queries(const RowsGeom& g, const AttnArgs& p, int qb, int slot)
{
    const int t0 = qb * g.Qb, t1 = std::min(p.S, t0 + g.Qb);
    const bool win = slot < g.n_wt;
    const int i0 = (win ? slot : slot - g.n_wt) * g.TR;
    if (win) {
        if (i0 >= g.WB) return -1;
        const int lo = t0 - p.W + 1 + i0, hi = t0 - p.W + 1 + std::min(i0 + g.TR, g.WB);
        return std::max(0, std::min(t1, hi + p.W - 1) - std::max(t0, lo));
    }
    const int nvmax = std::min(t1 / p.r, p.nc);
    if (i0 >= nvmax) return -1;
    return std::max(0, t1 - std::max(t0, (i0 + 1) * p.r - 1));
}

// Cost model of a schedule: a unit costs its queries plus a fixed overhead
// (row loads, pipeline fill, partial writes) in query steps; one workgroup
// per CU; each XCD (32 CUs on MI355X) hands its units, in order, to the
// first free CU.  Returns the finishing time of the last CU.
constexpr int N_XCD = 8, CU_PER_XCD = 32;
constexpr double UNIT_OVERHEAD = 2.0;

double rows_makespan(const std::vector<double> (&lists)[N_XCD])
{
    double worst = 0.0;
    for (int x = 0; x < N_XCD; ++x) {
        std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
        for (int i = 0; i < CU_PER_XCD; ++i) cu.push(0.0);
        double last = 0.0;
        for (const double c : lists[x]) {
            const double t = cu.top() + c;
            cu.pop();
            cu.push(t);
            last = std::max(last, t);
        }
        worst = std::max(worst, last);
    }
    return worst;
}

double unit_cost(int queries) { return queries < 0 ? 0.0 : queries + UNIT_OVERHEAD; }

// the closed-form round-robin schedule of the kernel (nmap = 0)
double rows_roundrobin_makespan(const RowsGeom& g, const AttnArgs& p)
{
    const int ntiles = g.n_wt + g.n_ct, nblk = p.b * g.nqb;
    const int64_t grid = (int64_t)(nblk + 7) / 8 * 8 * ntiles;
    std::vector<double> lists[N_XCD];
    for (int64_t lin = 0; lin < grid; ++lin) {
        const int xcd = (int)(lin & 7), kx = (int)(lin >> 3);
        const int qbi = (kx / ntiles) * 8 + xcd;
        if (qbi >= nblk) continue;
        lists[xcd].push_back(unit_cost(rows_unit_queries(g, p, g.nqb - 1 - qbi % g.nqb, kx % ntiles)));
    }
    return rows_makespan(lists);
}

// A table schedule: query blocks, heaviest first, each to the XCD with the
// fewest live units so far (then the least work); each XCD runs its units
// longest first.  Returns false when the table would not fit.
bool rows_table_plan(RowsGeom& g, const AttnArgs& p, double& makespan)
{
    const int ntiles = g.n_wt + g.n_ct, nblk = p.b * g.nqb;
    if ((int64_t)nblk * ntiles > ROWS_MAP_MAX) return false;
    struct Unit { int code; double cost; };
    std::vector<std::vector<Unit>> blk(nblk);
    std::vector<std::pair<double, int>> order;
    for (int qbi = 0; qbi < nblk; ++qbi) {
        double tot = 0.0;
        for (int slot = 0; slot < ntiles; ++slot) {
            const int n = rows_unit_queries(g, p, g.nqb - 1 - qbi % g.nqb, slot);
            blk[qbi].push_back({qbi * ntiles + slot, unit_cost(n)});
            tot += unit_cost(n);
        }
        order.push_back({-tot, qbi});
    }
    std::stable_sort(order.begin(), order.end());
    std::vector<Unit> per[N_XCD];
    int live[N_XCD] = {};
    double work[N_XCD] = {};
    for (const auto& o : order) {
        int best = 0;
        for (int x = 1; x < N_XCD; ++x)
            if (live[x] < live[best] || (live[x] == live[best] && work[x] < work[best])) best = x;
        for (const Unit& u : blk[o.second]) {
            per[best].push_back(u);
            live[best] += u.cost > 0.0;
            work[best] += u.cost;
        }
    }
    size_t len = 0;
    std::vector<double> lists[N_XCD];
    for (int x = 0; x < N_XCD; ++x) {
        std::stable_sort(per[x].begin(), per[x].end(), [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
        for (const Unit& u : per[x]) lists[x].push_back(u.cost);
        len = std::max(len, per[x].size());
    }
    if (len * N_XCD > (size_t)ROWS_MAP_MAX) return false;
    makespan = rows_makespan(lists);
    g.nmap = (int)(len * N_XCD);
    for (int i = 0; i < g.nmap; ++i) {
        const int x = i % N_XCD, k = i / N_XCD;
        g.map[i] = k < (int)per[x].size() ? (uint16_t)per[x][k].code : ROWS_IDLE;
    }
    return true;
}

}  // namespace

// Query block length and schedule of the key-stationary kernel.  They depend
// on the dimensions only (never on which optional inputs are given), so the
// workspace size a caller queries is the one the call uses.  The default is
// 32 queries (doubled while the partial rows would exceed 1 GiB; 128 for the
// window-free ratio-1 path) with the round-robin schedule; with a window,
// block lengths of 16..128 with a balanced table are tried, and the one with
// the shortest modelled finishing time wins.  Results are cached per shape (at
// most 64 shapes; the cache is emptied when it is full).
RowsGeom rows_geometry(const AttnArgs& p)
{
    using Key = std::array<int, 7>;
    static std::mutex mu;
    static std::map<Key, RowsGeom> cache;
    const Key key{p.b, p.S, p.H, p.D, p.W, p.r, p.nc};
    {
        std::lock_guard<std::mutex> lk(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int qb = (p.W == 0 && p.r == 1) ? 128 : 32;
    while (qb < 1024 && rows_partial_floats(p, qb) * 4 > ((int64_t)1 << 30)) qb *= 2;
    RowsGeom g{};
    rows_layout(g, p, qb);
    if (p.W > 0) {
        double best = rows_roundrobin_makespan(g, p);
        RowsGeom cand{};
        for (int q = 16; q <= 128; ++q) {
            if (rows_partial_floats(p, q) * 4 > ((int64_t)1 << 30)) continue;
            rows_layout(cand, p, q);
            double m;
            if (rows_table_plan(cand, p, m) && m < best) {
                best = m;
                g = cand;
            }
        }
    }
    std::lock_guard<std::mutex> lk(mu);
    if (cache.size() >= 64) cache.clear();      // bounded: a long-running caller with many shapes
    cache.emplace(key, g);
    return g;
}

template <typename T, int D, int HT, int KSP>
hipError_t launch_query_k(const AttnArgs& p, bool dq, float* delta, float* csink, hipStream_t st)
{
    const int gper = (p.H + 16 * HT - 1) / (16 * HT);
    int G = gper <= 1 ? 1 : (gper <= 2 ? 2 : 4);
    // wide rows with few heads: fewer queries per workgroup so the tiles fit
    // (the extra waves hold no head and only help gather rows)
    while (G < 4 && (size_t)(4 / G) * 2 * chunk_bytes<T, D>() > (size_t)ATTN_LDS_LIMIT) G *= 2;
    // a query whose heads need two waves runs alone in its workgroup (d <=
    // 128): each chunk barrier then couples only the waves that share the
    // tile, and no workgroup runs extra rounds for a longer neighbour
    const int qpw = (G == 2 && D <= 128) ? 1 : 4 / G;
    // two round tiles per query of the workgroup, then (when they fit) the index rows
    const int rbytes = (G == 2 && !dq) ? round_bytes<T, D, 2, false>() : chunk_bytes<T, D>();
    static_assert(round_chunks<T, D, 1, false>() == 1 && round_chunks<T, D, 4, false>() == 1 &&
                  round_chunks<T, D, 2, true>() == 1, "two-chunk rounds: the forward with G == 2 only");
    size_t lds = (size_t)qpw * 2 * rbytes;
    if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    const size_t with_ids = lds + (size_t)qpw * p.kp * sizeof(int32_t);
    const int idx_lds = (p.idx && p.kp > 0 && with_ids <= (size_t)ATTN_LDS_LIMIT) ? 1 : 0;
    // the kernels read index rows from their LDS copy only (it always fits: K' <= 2048)
    if (p.c && p.idx && p.kp > 0 && !idx_lds) return hipErrorInvalidValue;
    if (idx_lds) lds = with_ids;
    // document bits: window slots, plus every block in dense mode
    int okw = 0;
    if (p.doc) {
        const int nbits = min(p.W, p.S) + (p.c && !p.idx ? p.nc : 0);
        okw = (nbits + 63) / 64 * 2;
        lds += (size_t)qpw * okw * sizeof(uint32_t);
        if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    }
    auto go = [&](auto kern, int qpw_) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        dim3 grid((p.S + qpw_ - 1) / qpw_, p.b);
        TimedLaunch tl(dq ? K_ATTN_DQ : K_ATTN_FWD, st);
        hipLaunchKernelGGL(kern, grid, dim3(64 * G * qpw_), lds, st, p, delta, csink, idx_lds, okw);
        return hipGetLastError();
    };
    if (dq) {
        switch (G) {
        case 1: return go(attn_query_kernel<T, D, HT, 1, true, KSP>, 4);
        case 2: return go(attn_query_kernel<T, D, HT, 2, true, KSP>, qpw);
        default: return go(attn_query_kernel<T, D, HT, 4, true, KSP>, 1);
        }
    }
    switch (G) {
    case 1: return go(attn_query_kernel<T, D, HT, 1, false, KSP>, 4);
    case 2: return go(attn_query_kernel<T, D, HT, 2, false, KSP>, qpw);
    default: return go(attn_query_kernel<T, D, HT, 4, false, KSP>, 1);
    }
}

// packed [k | v] rows of 128 + 128 channels (the grouped-query path) skip
// their zero halves
template <typename T, int D, int HT>
hipError_t launch_query(const AttnArgs& p, bool dq, float* delta, float* csink, hipStream_t st)
{
    if constexpr (sizeof(T) == 2 && D == 256) {
        if (p.dsplit == 128) return launch_query_k<T, D, HT, 4>(p, dq, delta, csink, st);
    }
    return launch_query_k<T, D, HT, 0>(p, dq, delta, csink, st);
}

template <typename T>
hipError_t query_dispatch(const AttnArgs& p, bool dq, float* delta, float* csink, hipStream_t st)
{
    switch (p.D) {
    case 64:
        return p.H <= 16 ? launch_query<T, 64, 1>(p, dq, delta, csink, st) : launch_query<T, 64, 2>(p, dq, delta, csink, st);
    case 128:
        return p.H <= 16 ? launch_query<T, 128, 1>(p, dq, delta, csink, st)
                         : launch_query<T, 128, 2>(p, dq, delta, csink, st);
    case 256:
        if constexpr (sizeof(T) == 2) return launch_query<T, 256, 1>(p, dq, delta, csink, st);
        return hipErrorInvalidValue;
    case 512:   // fp32 rows of 512 exceed the on-chip tile (rejected at the boundary)
        if constexpr (sizeof(T) == 2) return launch_query<T, 512, 1>(p, dq, delta, csink, st);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

// the fixed-order reductions: dkv / dc rows (when gradients are requested) and dsink
template <int D>
hipError_t launch_reduce(const AttnArgs& p, const RowsGeom& geo, float* ws, hipStream_t st)
{
    const int64_t threads = p.dq ? (int64_t)p.b * (p.S + (p.c ? p.nc : 0)) * (D / 4) : 0;
    const int row_blocks = (int)((threads + 255) / 256);
    const int blocks = row_blocks + (p.sink && p.dsink ? p.H : 0);
    if (blocks == 0) return hipSuccess;
    TimedLaunch tl(K_ATTN_REDUCE, st);
    hipLaunchKernelGGL(attn_reduce_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, p, geo, (const float*)ws,
                       row_blocks);
    return hipGetLastError();
}

template <typename T, int D, int QS, int KSP>
hipError_t launch_rows_qk(const AttnArgs& p, const RowsGeom& geo, float* ws, hipStream_t st)
{
    constexpr int RW = rows_per_wave_t<T, D>(), NW = rows_waves_t<T, D>();
    const size_t lds = rows_lds_base<T, D, QS>() + (rows_tile_in_lds<T, D>() ? rows_lds_tile<T, D>() : 0) +
                       rows_lds_index<QS>();
    if (lds > (size_t)ATTN_LDS_LIMIT) return hipErrorInvalidValue;
    auto kern = attn_rows_kernel<T, D, RW, NW, QS, KSP>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int ntiles = geo.n_wt + (p.c ? geo.n_ct : 0);
    const int64_t groups = ((int64_t)p.b * geo.nqb + 7) / 8;     // rounds of 8 query blocks
    dim3 grid((unsigned)(geo.nmap > 0 ? geo.nmap : groups * 8 * ntiles));
    {
        TimedLaunch tl(K_ATTN_ROWS, st);
        hipLaunchKernelGGL(kern, grid, dim3(64 * NW), lds, st, p, geo, ws, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return launch_reduce<D>(p, geo, ws, st);
}

// Queries stacked in the 64 head slots: for the window-free path with an
// index list and at most 16 heads per query (d = 256 only, where the
// grouped-query path runs), 64 / (heads rounded up to a power of two >= 4)
// consecutive queries share one pass over the tile's rows.
template <typename T, int D, int QS>
hipError_t launch_rows_qs(const AttnArgs& p, const RowsGeom& geo, float* ws, hipStream_t st)
{
    if constexpr (sizeof(T) == 2 && D == 256) {
        if (p.dsplit == 128) return launch_rows_qk<T, D, QS, 4>(p, geo, ws, st);
    }
    return launch_rows_qk<T, D, QS, 0>(p, geo, ws, st);
}

template <typename T, int D>
hipError_t launch_rows(const AttnArgs& p, const RowsGeom& geo, float* ws, hipStream_t st)
{
    if constexpr (sizeof(T) == 2 && D == 256) {
        // the same test as attn_bwd_stacks_queries
        if (p.W == 0 && p.idx && p.H <= 16 && geo.Qb % 16 == 0) {
            if (p.H <= 4) return launch_rows_qs<T, D, 16>(p, geo, ws, st);
            if (p.H <= 8) return launch_rows_qs<T, D, 8>(p, geo, ws, st);
            return launch_rows_qs<T, D, 4>(p, geo, ws, st);
        }
    }
    return launch_rows_qs<T, D, 1>(p, geo, ws, st);
}

template <typename T>
hipError_t rows_dispatch(const AttnArgs& p, const RowsGeom& geo, float* ws, hipStream_t st)
{
    switch (p.D) {
    case 64: return launch_rows<T, 64>(p, geo, ws, st);
    case 128: return launch_rows<T, 128>(p, geo, ws, st);
    case 256:
        if constexpr (sizeof(T) == 2) return launch_rows<T, 256>(p, geo, ws, st);
        return hipErrorInvalidValue;
    case 512:
        if constexpr (sizeof(T) == 2) return launch_rows<T, 512>(p, geo, ws, st);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

// Selection bitmap of the index rows: one workgroup per (query, batch) sets
// the bits of the query's valid entries in LDS (an entry whose bit is already
// set is a repeat), then writes the row of words and the repeat flag.
__global__ __launch_bounds__(256) void selmap_kernel(const int32_t* __restrict__ idx, uint32_t* __restrict__ map,
                                                     int S, int kp, int r, int nc, int selw)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint32_t* bits = reinterpret_cast<uint32_t*>(smem);
    __shared__ uint32_t rep;
    const int t = blockIdx.x, nw = selw - 1;
    const int64_t row = (int64_t)blockIdx.y * S + t;
    for (int i = threadIdx.x; i < nw; i += 256) bits[i] = 0u;
    if (threadIdx.x == 0) rep = 0u;
    __syncthreads();
    const int nv = min((t + 1) / r, nc);
    const int32_t* irow = idx + row * kp;
    for (int s = threadIdx.x; s < kp; s += 256) {
        const int j = irow[s];
        if (j >= 0 && j < nv) {
            const uint32_t bit = 1u << (j & 31);
            if (atomicOr(&bits[j >> 5], bit) & bit) atomicOr(&rep, 1u);
        }
    }
    __syncthreads();
    uint32_t* out = map + row * selw;
    for (int i = threadIdx.x; i < nw; i += 256) out[i] = bits[i];
    if (threadIdx.x == 0) out[nw] = rep;
}

}  // namespace

int selmap_words(const AttnArgs& p)
{
    const int64_t w = ((int64_t)p.nc + 31) / 32 + 1;
    return (w - 1) * 4 <= 64 * 1024 ? (int)w : 0;
}

hipError_t build_selmap(const AttnArgs& p, uint32_t* map, hipStream_t st)
{
    const int w = selmap_words(p);
    if (!p.idx || w == 0 || p.b > 65535) return hipErrorInvalidValue;
    if (p.S == 0) return hipSuccess;
    hipLaunchKernelGGL(selmap_kernel, dim3((unsigned)p.S, (unsigned)p.b), dim3(256), (size_t)(w - 1) * 4, st, p.idx, map,
                       p.S, p.kp, p.r, p.nc, w);
    return hipGetLastError();
}

bool attn_bwd_stacks_queries(const AttnArgs& p, bool bf16)
{
    return bf16 && p.D == 256 && p.W == 0 && p.idx && p.H <= 16 && rows_geometry(p).Qb % 16 == 0;
}

int attn_bwd_query_block(const AttnArgs& p) { return rows_geometry(p).Qb; }

size_t attn_bwd_workspace_bytes(const AttnArgs& p)
{
    const RowsGeom g = rows_geometry(p);
    const int64_t floats = g.comp_off + (int64_t)p.b * g.nqb * p.nc * p.D;
    return (size_t)floats * 4;
}

// ----------------------------------------------- the backward's fixed scratch
// For callers that cannot allocate (graph capture, serving loops): the
// backward's workspace in a file-scope device array of ATTN_BWD_SCRATCH_BYTES,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: the device address of each GPU's copy comes
// from hipGetSymbolAddress, once per device with that device current.
namespace {
__device__ __align__(256) char scratch[ATTN_BWD_SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
}  // namespace

hipError_t attn_bwd_scratch(void** ptr)
{
    static std::mutex mu;
    static void* addr[SCRATCH_MAX_DEVICES] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t attn_fwd(const AttnArgs& p, bool bf16, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    return bf16 ? query_dispatch<bf16_t>(p, false, nullptr, nullptr, st)
                : query_dispatch<float>(p, false, nullptr, nullptr, st);
}

// ws: at least attn_bwd_workspace_bytes(p) bytes.  Delta (b*S*H floats) comes
// first, then the window partials, then the compressed partials.
hipError_t attn_bwd(const AttnArgs& p, bool bf16, float* ws, hipStream_t st)
{
    if (p.S == 0) return hipSuccess;
    const RowsGeom geo = rows_geometry(p);
    float* csink = (p.sink && p.dsink) ? ws + geo.sink_off : nullptr;
    hipError_t e = bf16 ? query_dispatch<bf16_t>(p, true, ws, csink, st) : query_dispatch<float>(p, true, ws, csink, st);
    if (e != hipSuccess) return e;
    if (!p.dq) {                                   // dsink only
        switch (p.D) {
        case 64: return launch_reduce<64>(p, geo, ws, st);
        case 128: return launch_reduce<128>(p, geo, ws, st);
        case 256: return launch_reduce<256>(p, geo, ws, st);
        default: return launch_reduce<512>(p, geo, ws, st);
        }
    }
    return bf16 ? rows_dispatch<bf16_t>(p, geo, ws, st) : rows_dispatch<float>(p, geo, ws, st);
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
