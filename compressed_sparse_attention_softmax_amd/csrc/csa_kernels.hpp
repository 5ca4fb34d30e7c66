// csa_kernels.hpp -- host-side launch interface of the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// dynamic LDS budget per workgroup on gfx950 (160 KiB per CU)
constexpr int INDEX_LDS_LIMIT = 160 * 1024;
constexpr int ATTN_LDS_LIMIT = 160 * 1024;

struct CompressArgs {
    const void* x;
    const void* z;
    int zc;
    void* c;
    float* c32;
    const float* dc;
    float* dx;
    float* dz;
    int b, S, D, r, L, nc;
    // epilogue: RMS norm weight [D] (nullptr: no norm), rotated trailing channels (0: none)
    const float* norm_w;
    float eps;
    int rope_dim;
    float rope_base;
    float* dnorm_w;       // [D] weight gradient (backward; nullptr: not wanted)
    float* ws;            // backward workspace when the epilogue is on
    // element strides (batch, token) of x and dx, and of z and dz
    int64_t xsb, xss, zsb, zss;
    void set_contiguous() { xsb = (int64_t)S * D; xss = D; zsb = (int64_t)S * zc; zss = zc; }
};

struct IndexArgs {
    const void* qi;
    const void* ki;
    const float* w;
    const int32_t* doc;   // [b, S] document ids, or nullptr (one document)
    int32_t* idx;
    float* score;
    int b, S, HI, DI, r, nc, kp;
    // element strides: q_i (batch, token, head), k_i (batch, block), w (batch, token)
    int64_t qsb, qss, qsh, ksb, kss, wsb, wss;
    void set_contiguous()
    {
        qsh = DI; qss = (int64_t)HI * DI; qsb = (int64_t)S * HI * DI;
        kss = DI; ksb = (int64_t)nc * DI;
        wss = HI; wsb = (int64_t)S * HI;
    }
};

struct AttnArgs {
    const void* q;
    const void* kv;
    const void* c;        // nullptr: window only
    const int32_t* idx;   // nullptr: every valid compressed row
    const float* sink;    // nullptr: no sink
    const int32_t* doc;   // [b, S] document ids, or nullptr (one document)
    float scale;
    void* out;
    float* lse;
    const void* dout;
    void* dq;
    float* dkv;
    float* dc;
    float* dsink;
    int b, S, H, D, W, r, nc, kp;
    // rows packed as [k | v] with q = [q | 0] and dO = [0 | dO] (the
    // grouped-query path): the first dsplit channels are the key half; the
    // kernels skip the products with a zero half (0: no packing)
    int dsplit;
    // optional selection bitmap of the index rows (built by build_selmap):
    // row (b, t) holds selw words, bit j of the first selw - 1 words set when
    // a valid entry of idx[b, t] names row j, and a last word that is nonzero
    // when such an entry repeats.  nullptr: the kernels scan the index rows.
    const uint32_t* selmap;
    int selw;
    // element strides: q-like tensors (q, out, dout, dq) along b, sequence,
    // head; kv-like (kv, dkv) along b and sequence; lse along b and sequence
    // (the last dimension is always contiguous).  set_contiguous() gives the
    // batch-major layout.
    int64_t qsb, qst, qsh, kvsb, kvst, lsb, lst;
    void set_contiguous()
    {
        qsh = D; qst = (int64_t)H * D; qsb = (int64_t)S * H * D;
        kvst = D; kvsb = (int64_t)S * D;
        lst = H; lsb = (int64_t)S * H;
    }
};

// Indexer distillation loss (teacher from the attention LSE, KL over the
// selected blocks) and its gradients into q_i, w and k_i.
struct LossArgs {
    const void* q;        // [b, S, H, D] attention queries
    const void* c;        // [b, nc, D] compressed rows
    const float* lse;     // [b, S, H] attention forward LSE
    const void* qi;       // [b, S, HI, DI]
    const void* ki;       // [b, nc, DI]
    const float* w;       // [b, S, HI]
    const int32_t* idx;   // [b, S, kp] selected blocks
    const float* score;   // [b, S, kp] their indexer scores
    float scale;
    const float* dkl;     // [b, S] upstream gradient of each row's KL (nullptr: forward only)
    float* kl;            // [b, S] or nullptr
    void* dqi;            // [b, S, HI, DI] (dtype) or nullptr (with dw, dki)
    float* dw;            // [b, S, HI]
    float* dki;           // [b, nc, DI]
    int b, S, H, D, HI, DI, r, nc, kp;
    // queries [t_begin, t_begin + t_count) of this launch (the dense form
    // runs the queries chunk by chunk; the selected form in one launch)
    int t_begin, t_count;
    // dense warm-up form (every valid block is the support): floats per
    // workspace row of a query; 0: the selected form
    int dense_ld;
    int dk_accumulate;    // the reduction adds into dk_i instead of overwriting it
};

// Simplified DSA over grouped-query attention: attention over the selected
// keys only, query head h reading key/value head h / (H / HKV).
struct GqaArgs {
    const void* q;        // [b, S, H, DK]
    const void* k;        // [b, S, HKV, DK]
    const void* v;        // [b, S, HKV, DV]
    const int32_t* idx;   // [b, S, kp] selected keys (valid: 0 <= j <= t)
    float scale;
    void* out;            // [b, S, H, DV]
    float* lse;           // [b, S, H]
    const void* dout;     // backward: [b, S, H, DV]
    void* dq;             // [b, S, H, DK] (dtype)
    float* dk;            // [b, S, HKV, DK]
    float* dv;            // [b, S, HKV, DV]
    int b, S, H, HKV, DK, DV, kp;
};

hipError_t compress_fwd(const CompressArgs& p, bool bf16, hipStream_t st);
hipError_t compress_bwd(const CompressArgs& p, bool bf16, hipStream_t st);
size_t compress_bwd_workspace_bytes(const CompressArgs& p);
hipError_t index_topk(const IndexArgs& p, bool bf16, hipStream_t st);
int index_topk_cap(const IndexArgs& p, bool bf16);
size_t topk_lds_bytes(int DI, int elem, int cap);
hipError_t attn_fwd(const AttnArgs& p, bool bf16, hipStream_t st);
hipError_t attn_bwd(const AttnArgs& p, bool bf16, float* ws, hipStream_t st);
size_t attn_bwd_workspace_bytes(const AttnArgs& p);
// consecutive queries per block of the backward's fixed-order row reduction
int attn_bwd_query_block(const AttnArgs& p);
// the backward's fixed scratch (a device array, one copy per GPU): its bytes,
// and the address of the current device's copy (looked up once per device)
constexpr size_t ATTN_BWD_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t attn_bwd_scratch(void** ptr);
// words per selection-bitmap row for p (0: too wide to build on chip)
int selmap_words(const AttnArgs& p);
// map: p.b * p.S * selmap_words(p) words; fills it from p.idx
hipError_t build_selmap(const AttnArgs& p, uint32_t* map, hipStream_t st);
// true when the backward's key-stationary kernel stacks queries (and then
// reads p.selmap when it is set)
bool attn_bwd_stacks_queries(const AttnArgs& p, bool bf16);
hipError_t indexer_loss(const LossArgs& p, bool bf16, float* ws, hipStream_t st);
size_t indexer_loss_workspace_bytes(const LossArgs& p);
// dense warm-up form: the bytes its plan uses within `budget` (at least the
// smallest plan), and the call on a workspace of ws_bytes (the plan fitting it)
size_t indexer_loss_dense_workspace_bytes(const LossArgs& p, size_t budget);
hipError_t indexer_loss_dense(const LossArgs& p, bool bf16, float* ws, size_t ws_bytes, hipStream_t st);
size_t dsa_gqa_workspace_bytes(const GqaArgs& p, bool bf16, bool bwd);
hipError_t dsa_gqa_fwd(const GqaArgs& p, bool bf16, void* ws, hipStream_t st);
hipError_t dsa_gqa_bwd(const GqaArgs& p, bool bf16, void* ws, hipStream_t st);
hipError_t zero_fill(float* p, size_t n, hipStream_t st);

}  // namespace csa
