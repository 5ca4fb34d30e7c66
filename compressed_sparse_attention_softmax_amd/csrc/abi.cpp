// abi.cpp -- the extern "C" entry points of libcsa (declared in include/csa.h).
//
// Each entry point validates every argument before touching the HIP runtime,
// records a message for csa_last_error() on failure, and enqueues the kernels
// on the caller's stream.  Every element of a gradient output is written by a
// kernel (a fill kernel where nothing else writes it; no memset nodes, so a
// caller may capture the calls into a graph).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <string>
#include <utility>
#include <vector>

#include "csa.h"
#include "csa_kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return CSA_OK;
}

int hip_status(hipError_t e, const char* where)
{
    if (e == hipSuccess) return ok();
    return fail(CSA_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool supported_d(int d) { return d == 64 || d == 128 || d == 512; }

// Every tensor base pointer of the CSA calls must be 16-byte aligned: the
// kernels move rows in 16-byte pieces (and fp32 rows in float4s).  NULL
// pointers are not checked here (each call decides which may be NULL).
typedef std::pair<const char*, const void*> named_ptr;
int check_aligned(const char* fn, std::initializer_list<named_ptr> ptrs)
{
    for (const named_ptr& p : ptrs)
        if (p.second && (reinterpret_cast<uintptr_t>(p.second) & 15))
            return fail(CSA_ERR_ARG, "%s: %s is not 16-byte aligned", fn, p.first);
    return CSA_OK;
}

int check_common(const csa_dims* dm, int dtype, const char* fn)
{
    if (!dm) return fail(CSA_ERR_ARG, "%s: dims is NULL", fn);
    if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (dm->b < 1 || dm->sq < 1) return fail(CSA_ERR_ARG, "%s: b=%d sq=%d must be >= 1", fn, dm->b, dm->sq);
    return CSA_OK;
}

int check_compress_dims(const csa_dims* dm, int z_channels, const char* fn)
{
    if (dm->ratio < 1 || dm->span < 1)
        return fail(CSA_ERR_ARG, "%s: ratio=%d span=%d must be >= 1", fn, dm->ratio, dm->span);
    if (!supported_d(dm->d)) return fail(CSA_ERR_UNSUPPORTED, "%s: d=%d not in {64,128,512}", fn, dm->d);
    if (z_channels != 1 && z_channels != dm->d)
        return fail(CSA_ERR_SHAPE, "%s: z_channels=%d must be 1 or d=%d", fn, z_channels, dm->d);
    return CSA_OK;
}

csa::CompressArgs compress_args(const csa_dims* dm, const void* x, const void* z, int zc)
{
    csa::CompressArgs a{};
    a.x = x; a.z = z; a.zc = zc;
    a.b = dm->b; a.S = dm->sq; a.D = dm->d; a.r = dm->ratio; a.L = dm->span;
    a.nc = dm->sq / dm->ratio;
    a.set_contiguous();
    return a;
}

int kprime(const csa_dims* dm) { return dm->topk < dm->sq / dm->ratio ? dm->topk : dm->sq / dm->ratio; }

int check_attn(const csa_dims* dm, int dtype, const void* q, const void* kv, const void* c,
               const int32_t* idx, float scale, const char* fn)
{
    if (!q || !kv) return fail(CSA_ERR_ARG, "%s: q and kv must be non-NULL", fn);
    if (!supported_d(dm->d)) return fail(CSA_ERR_UNSUPPORTED, "%s: d=%d not in {64,128,512}", fn, dm->d);
    if (dm->d == 512 && dtype == CSA_F32)
        return fail(CSA_ERR_UNSUPPORTED, "%s: fp32 with d=512 exceeds the on-chip row tile", fn);
    if (dm->h < 1) return fail(CSA_ERR_ARG, "%s: h=%d must be >= 1", fn, dm->h);
    if (dm->h > 64) return fail(CSA_ERR_UNSUPPORTED, "%s: h=%d > 64", fn, dm->h);
    if (dm->window < 1) return fail(CSA_ERR_ARG, "%s: window=%d must be >= 1", fn, dm->window);
    if (!std::isfinite(scale)) return fail(CSA_ERR_ARG, "%s: scale is not finite", fn);
    if (c) {
        if (dm->ratio < 1) return fail(CSA_ERR_ARG, "%s: ratio=%d must be >= 1", fn, dm->ratio);
        if (idx && dm->topk < 1) return fail(CSA_ERR_ARG, "%s: topk=%d must be >= 1 with idx", fn, dm->topk);
    } else if (idx) {
        return fail(CSA_ERR_ARG, "%s: idx given without compressed rows c", fn);
    }
    return CSA_OK;
}

csa::AttnArgs attn_args(const csa_dims* dm, const void* q, const void* kv, const void* c,
                        const int32_t* idx, const int32_t* doc_ids, const float* sink, float scale)
{
    csa::AttnArgs a{};
    a.q = q; a.kv = kv; a.c = c; a.idx = c ? idx : nullptr; a.sink = sink; a.scale = scale;
    a.doc = doc_ids;
    a.b = dm->b; a.S = dm->sq; a.H = dm->h; a.D = dm->d; a.W = dm->window;
    a.r = c ? dm->ratio : 1;
    a.nc = c ? dm->sq / dm->ratio : 0;
    a.kp = (c && idx) ? kprime(dm) : 0;
    a.set_contiguous();
    return a;
}

// Element strides of the strided attention calls.  For each tensor family the
// axes of extent > 1 (plus the contiguous last axis of the row) must be laid
// out without overlap: sorted by stride, every stride is at least the previous
// stride times the previous extent, so no two elements share an address.
// q-like and kv-like strides are multiples of 16 bytes (rows stay aligned for
// the 16-byte loads); axes of extent 1 are not checked (never multiplied by
// anything but 0).
struct Axis { int64_t stride, extent; };

bool no_overlap(std::vector<Axis> ax)
{
    std::vector<Axis> live;
    for (const Axis& a : ax)
        if (a.extent > 1) live.push_back(a);
    std::sort(live.begin(), live.end(), [](const Axis& x, const Axis& y) { return x.stride < y.stride; });
    for (size_t i = 1; i < live.size(); ++i)
        if (live[i - 1].stride < 1 || live[i].stride < live[i - 1].stride * live[i - 1].extent) return false;
    return live.empty() || live[0].stride >= 1;
}

int check_strides(const csa_dims* dm, int dtype, const csa_attn_strides* st, const char* fn)
{
    if (!st) return CSA_OK;
    const int64_t e = dtype == CSA_BF16 ? 8 : 4;       // elements per 16 bytes
    const int64_t b = dm->b, s = dm->sq, h = dm->h, d = dm->d;
    const struct { int64_t v, n; const char* name; } al[] = {
        {st->q_b, b, "q_b"}, {st->q_s, s, "q_s"}, {st->q_h, h, "q_h"}, {st->kv_b, b, "kv_b"}, {st->kv_s, s, "kv_s"}};
    for (const auto& x : al)
        if (x.n > 1 && (x.v < 1 || x.v % e))
            return fail(CSA_ERR_ARG, "%s: stride %s = %lld must be a positive multiple of %lld elements", fn, x.name,
                        (long long)x.v, (long long)e);
    if (!no_overlap({{1, d}, {st->q_b, b}, {st->q_s, s}, {st->q_h, h}}))
        return fail(CSA_ERR_ARG, "%s: q strides (%lld, %lld, %lld) make rows overlap", fn, (long long)st->q_b,
                    (long long)st->q_s, (long long)st->q_h);
    if (!no_overlap({{1, d}, {st->kv_b, b}, {st->kv_s, s}}))
        return fail(CSA_ERR_ARG, "%s: kv strides (%lld, %lld) make rows overlap", fn, (long long)st->kv_b,
                    (long long)st->kv_s);
    if (!no_overlap({{1, h}, {st->lse_b, b}, {st->lse_s, s}}))
        return fail(CSA_ERR_ARG, "%s: lse strides (%lld, %lld) make rows overlap", fn, (long long)st->lse_b,
                    (long long)st->lse_s);
    return CSA_OK;
}

void apply_strides(csa::AttnArgs& a, const csa_attn_strides* st)
{
    if (!st) return;
    a.qsb = st->q_b; a.qst = st->q_s; a.qsh = st->q_h;
    a.kvsb = st->kv_b; a.kvst = st->kv_s;
    a.lsb = st->lse_b; a.lst = st->lse_s;
}

// One stride of a row-addressed tensor: positive, and a multiple of `mult`
// elements when its axis has more than one entry.
struct StrideCheck { int64_t v, n, mult; const char* name; };

int check_stride_list(std::initializer_list<StrideCheck> l, const char* fn)
{
    for (const auto& x : l)
        if (x.n > 1 && (x.v < 1 || x.v % x.mult))
            return fail(CSA_ERR_ARG, "%s: stride %s = %lld must be a positive multiple of %lld elements", fn, x.name,
                        (long long)x.v, (long long)x.mult);
    return CSA_OK;
}

// x / dx rows of d channels and z / dz rows of z_channels, strided by token
// and batch; rows that 16-byte loads read (x, and z with z_channels = d) keep
// 16-byte aligned strides
int check_compress_strides(const csa_dims* dm, int dtype, int zc, const csa_compress_strides* st, const char* fn)
{
    if (!st) return CSA_OK;
    const int64_t e = dtype == CSA_BF16 ? 8 : 4;
    const int64_t b = dm->b, s = dm->sq, d = dm->d;
    int rc = check_stride_list({{st->x_b, b, e, "x_b"}, {st->x_s, s, e, "x_s"},
                                {st->z_b, b, zc == 1 ? 1 : e, "z_b"}, {st->z_s, s, zc == 1 ? 1 : e, "z_s"}}, fn);
    if (rc) return rc;
    if (!no_overlap({{1, d}, {st->x_b, b}, {st->x_s, s}}))
        return fail(CSA_ERR_ARG, "%s: x strides (%lld, %lld) make rows overlap", fn, (long long)st->x_b,
                    (long long)st->x_s);
    if (!no_overlap({{1, zc}, {st->z_b, b}, {st->z_s, s}}))
        return fail(CSA_ERR_ARG, "%s: z strides (%lld, %lld) make rows overlap", fn, (long long)st->z_b,
                    (long long)st->z_s);
    return CSA_OK;
}

void apply_compress_strides(csa::CompressArgs& a, const csa_compress_strides* st)
{
    if (!st) return;
    a.xsb = st->x_b; a.xss = st->x_s; a.zsb = st->z_b; a.zss = st->z_s;
}

// q_i rows of idx_dim (by token, head, batch), k_i rows (by block, batch), w
// rows of idx_heads (by token, batch; ignored when there is no w); q_i and k_i
// rows are read with 16-byte loads
int check_index_strides(const csa_dims* dm, int dtype, const csa_index_strides* st, bool has_w, const char* fn)
{
    if (!st) return CSA_OK;
    const int64_t e = dtype == CSA_BF16 ? 8 : 4;
    const int64_t b = dm->b, s = dm->sq, hi = dm->idx_heads, di = dm->idx_dim, nc = dm->sq / dm->ratio;
    int rc = check_stride_list({{st->qi_b, b, e, "qi_b"}, {st->qi_s, s, e, "qi_s"}, {st->qi_h, hi, e, "qi_h"},
                                {st->ki_b, b, e, "ki_b"}, {st->ki_s, nc, e, "ki_s"},
                                {st->w_b, has_w ? b : 1, 1, "w_b"}, {st->w_s, has_w ? s : 1, 1, "w_s"}}, fn);
    if (rc) return rc;
    if (!no_overlap({{1, di}, {st->qi_b, b}, {st->qi_s, s}, {st->qi_h, hi}}))
        return fail(CSA_ERR_ARG, "%s: q_i strides (%lld, %lld, %lld) make rows overlap", fn, (long long)st->qi_b,
                    (long long)st->qi_s, (long long)st->qi_h);
    if (!no_overlap({{1, di}, {st->ki_b, b}, {st->ki_s, nc}}))
        return fail(CSA_ERR_ARG, "%s: k_i strides (%lld, %lld) make rows overlap", fn, (long long)st->ki_b,
                    (long long)st->ki_s);
    if (has_w && !no_overlap({{1, hi}, {st->w_b, b}, {st->w_s, s}}))
        return fail(CSA_ERR_ARG, "%s: w strides (%lld, %lld) make rows overlap", fn, (long long)st->w_b,
                    (long long)st->w_s);
    return CSA_OK;
}

void apply_index_strides(csa::IndexArgs& a, const csa_index_strides* st)
{
    if (!st) return;
    a.qsb = st->qi_b; a.qss = st->qi_s; a.qsh = st->qi_h;
    a.ksb = st->ki_b; a.kss = st->ki_s;
    a.wsb = st->w_b; a.wss = st->w_s;
}

int check_epilogue(const csa_dims* dm, const float* norm_w, float eps, int rope_dim, float base, const char* fn)
{
    if (norm_w && !(std::isfinite(eps) && eps >= 0.f))
        return fail(CSA_ERR_ARG, "%s: norm_eps=%g must be finite and >= 0", fn, (double)eps);
    if (rope_dim < 0 || rope_dim > dm->d || (rope_dim & 1))
        return fail(CSA_ERR_ARG, "%s: rope_dim=%d must be even and in [0, d=%d]", fn, rope_dim, dm->d);
    if (rope_dim > 0 && !(std::isfinite(base) && base > 0.f))
        return fail(CSA_ERR_ARG, "%s: rope_base=%g must be finite and > 0", fn, (double)base);
    return CSA_OK;
}

void set_epilogue(csa::CompressArgs& a, const float* norm_w, float eps, int rope_dim, float base)
{
    a.norm_w = norm_w; a.eps = eps; a.rope_dim = rope_dim; a.rope_base = base;
}

// the compressor and indexer calls, with optional element strides (NULL: contiguous)
int compress_call(const csa_dims* dm, const csa_compress_strides* st, int dtype, const void* x, const void* z,
                  int z_channels, const float* norm_w, float norm_eps, int rope_dim, float rope_base, void* c,
                  float* c32, void* stream, const char* fn)
{
    int rc = check_common(dm, dtype, fn);
    if (rc) return rc;
    if ((rc = check_compress_dims(dm, z_channels, fn))) return rc;
    if ((rc = check_epilogue(dm, norm_w, norm_eps, rope_dim, rope_base, fn))) return rc;
    if (!x || !z || (!c && dm->sq / dm->ratio > 0))
        return fail(CSA_ERR_ARG, "%s: x, z and c must be non-NULL", fn);
    if ((rc = check_aligned(fn, {{"x", x}, {"z", z}, {"norm_w", norm_w}, {"c", c}, {"c32", c32}})))
        return rc;
    if ((rc = check_compress_strides(dm, dtype, z_channels, st, fn))) return rc;
    csa::CompressArgs a = compress_args(dm, x, z, z_channels);
    apply_compress_strides(a, st);
    a.c = c; a.c32 = c32;
    set_epilogue(a, norm_w, norm_eps, rope_dim, rope_base);
    return hip_status(csa::compress_fwd(a, dtype == CSA_BF16, (hipStream_t)stream), fn);
}

int compress_bwd_call(const csa_dims* dm, const csa_compress_strides* st, int dtype, const void* x, const void* z,
                      int z_channels, const float* norm_w, float norm_eps, int rope_dim, float rope_base,
                      const float* dc, float* dx, float* dz, float* dnorm_w, void* ws, size_t ws_bytes, void* stream,
                      const char* fn)
{
    int rc = check_common(dm, dtype, fn);
    if (rc) return rc;
    if ((rc = check_compress_dims(dm, z_channels, fn))) return rc;
    if ((rc = check_epilogue(dm, norm_w, norm_eps, rope_dim, rope_base, fn))) return rc;
    if (!x || !z || (!dc && dm->sq / dm->ratio > 0) || !dx || !dz)
        return fail(CSA_ERR_ARG, "%s: x, z, dc, dx and dz must be non-NULL", fn);
    if (dnorm_w && !norm_w) return fail(CSA_ERR_ARG, "%s: dnorm_w given without norm_w", fn);
    if ((rc = check_aligned(fn, {{"x", x}, {"z", z}, {"norm_w", norm_w}, {"dc", dc}, {"dx", dx}, {"dz", dz},
                                 {"dnorm_w", dnorm_w}})))
        return rc;
    if ((rc = check_compress_strides(dm, dtype, z_channels, st, fn))) return rc;
    csa::CompressArgs a = compress_args(dm, x, z, z_channels);
    apply_compress_strides(a, st);
    a.dc = dc; a.dx = dx; a.dz = dz;
    set_epilogue(a, norm_w, norm_eps, rope_dim, rope_base);
    a.dnorm_w = dnorm_w;
    const size_t need = csa::compress_bwd_workspace_bytes(a);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        ws ? ws_bytes : (size_t)0);
        if (((uintptr_t)ws) & 15) return fail(CSA_ERR_ARG, "%s: workspace must be 16-byte aligned", fn);
    }
    a.ws = (float*)ws;
    return hip_status(csa::compress_bwd(a, dtype == CSA_BF16, (hipStream_t)stream), fn);
}

int index_topk_call(const csa_dims* dm, const csa_index_strides* st, int dtype, const void* q_i, const void* k_i,
                    const float* w, const int32_t* doc_ids, int32_t* idx, float* score, void* stream, const char* fn)
{
    int rc = check_common(dm, dtype, fn);
    if (rc) return rc;
    if (dm->ratio < 1) return fail(CSA_ERR_ARG, "%s: ratio=%d must be >= 1", fn, dm->ratio);
    if (dm->topk < 1) return fail(CSA_ERR_ARG, "%s: topk=%d must be >= 1", fn, dm->topk);
    if (dm->idx_heads < 1) return fail(CSA_ERR_ARG, "%s: idx_heads=%d must be >= 1", fn, dm->idx_heads);
    if (dm->idx_heads > 64) return fail(CSA_ERR_UNSUPPORTED, "%s: idx_heads=%d > 64", fn, dm->idx_heads);
    if (dm->idx_dim != 32 && dm->idx_dim != 64 && dm->idx_dim != 128)
        return fail(CSA_ERR_UNSUPPORTED, "%s: idx_dim=%d not in {32,64,128}", fn, dm->idx_dim);
    const int kp = kprime(dm);
    if (!q_i) return fail(CSA_ERR_ARG, "%s: q_i must be non-NULL", fn);
    // sq < ratio: no block exists, K' = 0, idx / score / k_i have no elements
    if (kp == 0) return ok();
    if (!k_i || !idx) return fail(CSA_ERR_ARG, "%s: k_i and idx must be non-NULL", fn);
    if (kp > 2048) return fail(CSA_ERR_UNSUPPORTED, "%s: K'=%d > 2048", fn, kp);
    if ((rc = check_aligned(fn, {{"q_i", q_i}, {"k_i", k_i}, {"w", w}, {"doc_ids", doc_ids}, {"idx", idx},
                                 {"score", score}})))
        return rc;
    if ((rc = check_index_strides(dm, dtype, st, w != nullptr, fn))) return rc;
    csa::IndexArgs a{};
    a.qi = q_i; a.ki = k_i; a.w = w; a.doc = doc_ids; a.idx = idx; a.score = score;
    a.b = dm->b; a.S = dm->sq; a.HI = dm->idx_heads; a.DI = dm->idx_dim; a.r = dm->ratio;
    a.nc = dm->sq / dm->ratio; a.kp = kp;
    a.set_contiguous();
    apply_index_strides(a, st);
    if (kp > 0 && csa::index_topk_cap(a, dtype == CSA_BF16) == 0)
        return fail(CSA_ERR_UNSUPPORTED, "%s: K'=%d does not fit the on-chip candidate buffer", fn, kp);
    return hip_status(csa::index_topk(a, dtype == CSA_BF16, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

int csa_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_err.c_str(); }

int csa_compress(const csa_dims* dm, int dtype, const void* x, const void* z, int z_channels, const float* norm_w,
                 float norm_eps, int rope_dim, float rope_base, void* c, float* c32, void* stream)
{
    return compress_call(dm, nullptr, dtype, x, z, z_channels, norm_w, norm_eps, rope_dim, rope_base, c, c32, stream,
                         "csa_compress");
}

int csa_compress_strided(const csa_dims* dm, const csa_compress_strides* strides, int dtype, const void* x,
                         const void* z, int z_channels, const float* norm_w, float norm_eps, int rope_dim,
                         float rope_base, void* c, float* c32, void* stream)
{
    return compress_call(dm, strides, dtype, x, z, z_channels, norm_w, norm_eps, rope_dim, rope_base, c, c32, stream,
                         "csa_compress_strided");
}

size_t csa_compress_bwd_workspace(const csa_dims* dm)
{
    if (!dm || dm->b < 1 || dm->sq < 1 || dm->ratio < 1 || !supported_d(dm->d)) return 0;
    csa::CompressArgs a = compress_args(dm, nullptr, nullptr, 1);
    a.rope_dim = 2;                      // the epilogue's layout
    return csa::compress_bwd_workspace_bytes(a);
}

int csa_compress_bwd(const csa_dims* dm, int dtype, const void* x, const void* z, int z_channels,
                     const float* norm_w, float norm_eps, int rope_dim, float rope_base, const float* dc, float* dx,
                     float* dz, float* dnorm_w, void* ws, size_t ws_bytes, void* stream)
{
    return compress_bwd_call(dm, nullptr, dtype, x, z, z_channels, norm_w, norm_eps, rope_dim, rope_base, dc, dx, dz,
                             dnorm_w, ws, ws_bytes, stream, "csa_compress_bwd");
}

int csa_compress_bwd_strided(const csa_dims* dm, const csa_compress_strides* strides, int dtype, const void* x,
                             const void* z, int z_channels, const float* norm_w, float norm_eps, int rope_dim,
                             float rope_base, const float* dc, float* dx, float* dz, float* dnorm_w, void* ws,
                             size_t ws_bytes, void* stream)
{
    return compress_bwd_call(dm, strides, dtype, x, z, z_channels, norm_w, norm_eps, rope_dim, rope_base, dc, dx, dz,
                             dnorm_w, ws, ws_bytes, stream, "csa_compress_bwd_strided");
}

size_t csa_index_topk_workspace(const csa_dims* dm)
{
    (void)dm;
    return 0;
}

int csa_index_topk(const csa_dims* dm, int dtype, const void* q_i, const void* k_i, const float* w,
                   const int32_t* doc_ids, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                   void* stream)
{
    (void)ws; (void)ws_bytes;
    return index_topk_call(dm, nullptr, dtype, q_i, k_i, w, doc_ids, idx, score, stream, "csa_index_topk");
}

int csa_index_topk_strided(const csa_dims* dm, const csa_index_strides* strides, int dtype, const void* q_i,
                           const void* k_i, const float* w, const int32_t* doc_ids, int32_t* idx, float* score,
                           void* ws, size_t ws_bytes, void* stream)
{
    (void)ws; (void)ws_bytes;
    return index_topk_call(dm, strides, dtype, q_i, k_i, w, doc_ids, idx, score, stream, "csa_index_topk_strided");
}

}  // extern "C"

namespace {

int attn_fwd_call(const csa_dims* dm, const csa_attn_strides* st, int dtype, const void* q, const void* kv,
                  const void* c, const int32_t* idx, const int32_t* doc_ids, const float* sink, float scale,
                  void* out, float* lse, void* stream, const char* fn)
{
    int rc = check_common(dm, dtype, fn);
    if (rc) return rc;
    if ((rc = check_attn(dm, dtype, q, kv, c, idx, scale, fn))) return rc;
    if ((rc = check_strides(dm, dtype, st, fn))) return rc;
    if (!out || !lse) return fail(CSA_ERR_ARG, "%s: out and lse must be non-NULL", fn);
    if ((rc = check_aligned(fn, {{"q", q}, {"kv", kv}, {"c", c}, {"idx", idx}, {"doc_ids", doc_ids},
                                 {"sink", sink}, {"out", out}, {"lse", lse}})))
        return rc;
    csa::AttnArgs a = attn_args(dm, q, kv, c, idx, doc_ids, sink, scale);
    apply_strides(a, st);
    a.out = out; a.lse = lse;
    return hip_status(csa::attn_fwd(a, dtype == CSA_BF16, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

int csa_sparse_attn_fwd(const csa_dims* dm, int dtype, const void* q, const void* kv, const void* c,
                        const int32_t* idx, const int32_t* doc_ids, const float* sink, float scale,
                        void* out, float* lse, void* stream)
{
    return attn_fwd_call(dm, nullptr, dtype, q, kv, c, idx, doc_ids, sink, scale, out, lse, stream,
                         "csa_sparse_attn_fwd");
}

int csa_sparse_attn_fwd_strided(const csa_dims* dm, const csa_attn_strides* strides, int dtype, const void* q,
                                const void* kv, const void* c, const int32_t* idx, const int32_t* doc_ids,
                                const float* sink, float scale, void* out, float* lse, void* stream)
{
    return attn_fwd_call(dm, strides, dtype, q, kv, c, idx, doc_ids, sink, scale, out, lse, stream,
                         "csa_sparse_attn_fwd_strided");
}

size_t csa_sparse_attn_bwd_workspace(const csa_dims* dm)
{
    if (!dm || dm->b < 1 || dm->sq < 1 || dm->h < 1 || dm->window < 1 || !supported_d(dm->d)) return 0;
    // the larger of the layouts with and without compressed rows
    csa::AttnArgs a{};
    a.b = dm->b; a.S = dm->sq; a.H = dm->h; a.D = dm->d; a.W = dm->window; a.r = 1; a.nc = 0;
    size_t w0 = csa::attn_bwd_workspace_bytes(a);
    if (dm->ratio >= 1) {
        a.r = dm->ratio;
        a.nc = dm->sq / dm->ratio;
        const size_t w1 = csa::attn_bwd_workspace_bytes(a);
        if (w1 > w0) w0 = w1;
    }
    return w0;
}

int csa_sparse_attn_bwd_query_block(const csa_dims* dm, int with_compressed)
{
    if (!dm || dm->b < 1 || dm->sq < 1 || dm->h < 1 || dm->window < 1 || !supported_d(dm->d)) return 0;
    if (with_compressed && dm->ratio < 1) return 0;
    csa::AttnArgs a{};
    a.b = dm->b; a.S = dm->sq; a.H = dm->h; a.D = dm->d; a.W = dm->window;
    a.r = with_compressed ? dm->ratio : 1;
    a.nc = with_compressed ? dm->sq / dm->ratio : 0;
    return csa::attn_bwd_query_block(a);
}

}  // extern "C"

namespace {

// validation and arguments of the attention backward (both entry points)
int attn_bwd_prepare(const csa_dims* dm, int dtype, const void* q, const void* kv, const void* c, const int32_t* idx,
                     const int32_t* doc_ids, const float* sink, float scale, const void* out, const float* lse,
                     const void* dout, void* dq, float* dkv, float* dc, float* dsink, const char* fn,
                     csa::AttnArgs& a, bool& noop, const csa_attn_strides* st = nullptr)
{
    noop = false;
    int rc = check_common(dm, dtype, fn);
    if (rc) return rc;
    if ((rc = check_attn(dm, dtype, q, kv, c, idx, scale, fn))) return rc;
    if ((rc = check_strides(dm, dtype, st, fn))) return rc;
    if (!out || !lse || !dout) return fail(CSA_ERR_ARG, "%s: out, lse and dout must be non-NULL", fn);
    // all-or-nothing gradient gate
    const bool want_c = c != nullptr;
    const bool any = dq || dkv || dc;
    if (!want_c && dc) return fail(CSA_ERR_ARG, "%s: dc given without compressed rows c", fn);
    if (any) {
        if (!dq) return fail(CSA_ERR_ARG, "%s: gradient gate: dq is NULL while other gradients are requested", fn);
        if (!dkv) return fail(CSA_ERR_ARG, "%s: gradient gate: dkv is NULL while other gradients are requested", fn);
        if (want_c && !dc) return fail(CSA_ERR_ARG, "%s: gradient gate: dc is NULL while other gradients are requested", fn);
    }
    if (dsink && !sink) return fail(CSA_ERR_ARG, "%s: dsink given without sink", fn);
    if ((rc = check_aligned(fn, {{"q", q}, {"kv", kv}, {"c", c}, {"idx", idx}, {"doc_ids", doc_ids},
                                 {"sink", sink}, {"out", out}, {"lse", lse}, {"dout", dout}, {"dq", dq},
                                 {"dkv", dkv}, {"dc", dc}, {"dsink", dsink}})))
        return rc;
    if (!any && !dsink) {
        noop = true;
        return ok();
    }
    a = attn_args(dm, q, kv, c, idx, doc_ids, sink, scale);
    apply_strides(a, st);
    a.out = const_cast<void*>(out); a.lse = const_cast<float*>(lse); a.dout = dout;
    a.dq = dq; a.dkv = dkv; a.dc = dc; a.dsink = dsink;
    return CSA_OK;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

int attn_bwd_call(const csa_dims* dm, const csa_attn_strides* strides, int dtype, const void* q, const void* kv,
                  const void* c, const int32_t* idx, const int32_t* doc_ids, const float* sink, float scale,
                  const void* out, const float* lse, const void* dout, void* dq, float* dkv, float* dc,
                  float* dsink, void* ws, size_t ws_bytes, void* stream, const char* fn)
{
    csa::AttnArgs a{};
    bool noop = false;
    int rc = attn_bwd_prepare(dm, dtype, q, kv, c, idx, doc_ids, sink, scale, out, lse, dout, dq, dkv, dc, dsink,
                              fn, a, noop, strides);
    if (rc || noop) return rc;
    const size_t need = csa::attn_bwd_workspace_bytes(a);
    if (!ws || ws_bytes < need)
        return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws ? ws_bytes : (size_t)0);
    if (((uintptr_t)ws) & 15) return fail(CSA_ERR_ARG, "%s: workspace must be 16-byte aligned", fn);
    return hip_status(csa::attn_bwd(a, dtype == CSA_BF16, (float*)ws, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

int csa_sparse_attn_bwd(const csa_dims* dm, int dtype, const void* q, const void* kv, const void* c,
                        const int32_t* idx, const int32_t* doc_ids, const float* sink, float scale, const void* out,
                        const float* lse, const void* dout, void* dq, float* dkv, float* dc,
                        float* dsink, void* ws, size_t ws_bytes, void* stream)
{
    return attn_bwd_call(dm, nullptr, dtype, q, kv, c, idx, doc_ids, sink, scale, out, lse, dout, dq, dkv, dc, dsink,
                         ws, ws_bytes, stream, "csa_sparse_attn_bwd");
}

int csa_sparse_attn_bwd_strided(const csa_dims* dm, const csa_attn_strides* strides, int dtype, const void* q,
                                const void* kv, const void* c, const int32_t* idx, const int32_t* doc_ids,
                                const float* sink, float scale, const void* out, const float* lse,
                                const void* dout, void* dq, float* dkv, float* dc, float* dsink, void* ws,
                                size_t ws_bytes, void* stream)
{
    return attn_bwd_call(dm, strides, dtype, q, kv, c, idx, doc_ids, sink, scale, out, lse, dout, dq, dkv, dc, dsink,
                         ws, ws_bytes, stream, "csa_sparse_attn_bwd_strided");
}

int csa_sparse_attn_bwd_noalloc(const csa_dims* dm, int dtype, const void* q, const void* kv, const void* c,
                                const int32_t* idx, const int32_t* doc_ids, const float* sink, float scale,
                                const void* out, const float* lse, const void* dout, void* dq, float* dkv,
                                float* dc, float* dsink, void* stream)
{
    csa::AttnArgs a{};
    bool noop = false;
    int rc = attn_bwd_prepare(dm, dtype, q, kv, c, idx, doc_ids, sink, scale, out, lse, dout, dq, dkv, dc, dsink,
                              "csa_sparse_attn_bwd_noalloc", a, noop);
    if (rc || noop) return rc;
    const size_t need = csa::attn_bwd_workspace_bytes(a);
    static_assert(csa::ATTN_BWD_SCRATCH_BYTES == (size_t)CSA_BWD_SCRATCH_BYTES, "header and library agree");
    if (need > csa::ATTN_BWD_SCRATCH_BYTES)
        return fail(CSA_ERR_UNSUPPORTED,
                    "csa_sparse_attn_bwd_noalloc: these dims need %zu bytes of scratch, more than the fixed %zu "
                    "(use csa_sparse_attn_bwd with a caller workspace)", need, csa::ATTN_BWD_SCRATCH_BYTES);
    void* scr = nullptr;
    hipError_t e = csa::attn_bwd_scratch(&scr);
    if (e != hipSuccess) return hip_status(e, "csa_sparse_attn_bwd_noalloc: scratch address");
    return hip_status(csa::attn_bwd(a, dtype == CSA_BF16, (float*)scr, (hipStream_t)stream),
                      "csa_sparse_attn_bwd_noalloc");
}

}  // extern "C"

namespace {

int check_loss(const csa_dims* dm, int dtype, const char* fn, bool dense = false)
{
    if (!supported_d(dm->d)) return fail(CSA_ERR_UNSUPPORTED, "%s: d=%d not in {64,128,512}", fn, dm->d);
    if (dm->d == 512 && dtype == CSA_F32)
        return fail(CSA_ERR_UNSUPPORTED, "%s: fp32 with d=512 exceeds the on-chip row tile", fn);
    if (dm->h < 1 || dm->h > 64) return fail(dm->h < 1 ? CSA_ERR_ARG : CSA_ERR_UNSUPPORTED, "%s: h=%d not in [1, 64]", fn, dm->h);
    if (dm->ratio < 1) return fail(CSA_ERR_ARG, "%s: ratio=%d must be >= 1", fn, dm->ratio);
    if (!dense && dm->topk < 1) return fail(CSA_ERR_ARG, "%s: topk=%d must be >= 1", fn, dm->topk);
    if (dm->idx_heads < 1 || dm->idx_heads > 64)
        return fail(dm->idx_heads < 1 ? CSA_ERR_ARG : CSA_ERR_UNSUPPORTED, "%s: idx_heads=%d not in [1, 64]", fn,
                    dm->idx_heads);
    if (dm->idx_dim != 32 && dm->idx_dim != 64 && dm->idx_dim != 128)
        return fail(CSA_ERR_UNSUPPORTED, "%s: idx_dim=%d not in {32,64,128}", fn, dm->idx_dim);
    if (!dense && kprime(dm) > 2048) return fail(CSA_ERR_UNSUPPORTED, "%s: K'=%d > 2048", fn, kprime(dm));
    return CSA_OK;
}

csa::LossArgs loss_args(const csa_dims* dm)
{
    csa::LossArgs a{};
    a.b = dm->b; a.S = dm->sq; a.H = dm->h; a.D = dm->d; a.HI = dm->idx_heads; a.DI = dm->idx_dim;
    a.r = dm->ratio; a.nc = dm->sq / dm->ratio; a.kp = kprime(dm);
    a.t_begin = 0; a.t_count = dm->sq;
    return a;
}

}  // namespace

extern "C" {

size_t csa_indexer_loss_workspace(const csa_dims* dm)
{
    if (!dm || dm->b < 1 || dm->sq < 1 || dm->ratio < 1 || dm->topk < 1) return 0;
    if (dm->idx_dim != 32 && dm->idx_dim != 64 && dm->idx_dim != 128) return 0;
    return csa::indexer_loss_workspace_bytes(loss_args(dm));
}

int csa_indexer_loss(const csa_dims* dm, int dtype, const void* q, const void* c, const float* lse,
                     const void* q_i, const void* k_i, const float* w, const int32_t* idx, const float* score,
                     float scale, const float* dkl, float* kl, void* dq_i, float* dw, float* dk_i, void* ws,
                     size_t ws_bytes, void* stream)
{
    int rc = check_common(dm, dtype, "csa_indexer_loss");
    if (rc) return rc;
    if ((rc = check_loss(dm, dtype, "csa_indexer_loss"))) return rc;
    if (!std::isfinite(scale)) return fail(CSA_ERR_ARG, "csa_indexer_loss: scale is not finite");
    // tensors with no elements (no compressed block yet: n_c = K' = 0) may be NULL
    const bool blocks = dm->sq / dm->ratio > 0;
    if (!q || !lse || (blocks && (!c || !idx || !score)))
        return fail(CSA_ERR_ARG, "csa_indexer_loss: q, c, lse, idx and score must be non-NULL");
    const bool any = dkl || dq_i || dw || dk_i;
    if (any) {
        if (!dkl || !dq_i || !dw || (blocks && !dk_i))
            return fail(CSA_ERR_ARG, "csa_indexer_loss: gradient gate: dkl, dq_i, dw and dk_i must all be given "
                                     "(or all be NULL)");
        if (!q_i || !w || (blocks && !k_i))
            return fail(CSA_ERR_ARG, "csa_indexer_loss: q_i, k_i and w must be non-NULL with gradients");
    }
    if ((rc = check_aligned("csa_indexer_loss", {{"q", q}, {"c", c}, {"lse", lse}, {"q_i", q_i}, {"k_i", k_i},
                                                 {"w", w}, {"idx", idx}, {"score", score}, {"dkl", dkl},
                                                 {"kl", kl}, {"dq_i", dq_i}, {"dw", dw}, {"dk_i", dk_i}})))
        return rc;
    if (!any && !kl) return ok();
    csa::LossArgs a = loss_args(dm);
    a.q = q; a.c = c; a.lse = lse; a.qi = q_i; a.ki = k_i; a.w = w; a.idx = idx; a.score = score;
    a.scale = scale; a.dkl = dkl; a.kl = kl; a.dqi = dq_i; a.dw = dw; a.dki = dk_i;
    if (any) {
        const size_t need = csa::indexer_loss_workspace_bytes(a);
        if (need > 0 && (!ws || ws_bytes < need))
            return fail(CSA_ERR_WORKSPACE, "csa_indexer_loss: workspace of %zu bytes needed, %zu given", need,
                        ws ? ws_bytes : (size_t)0);
        if (((uintptr_t)ws) & 15) return fail(CSA_ERR_ARG, "csa_indexer_loss: workspace must be 16-byte aligned");
    }
    return hip_status(csa::indexer_loss(a, dtype == CSA_BF16, (float*)ws, (hipStream_t)stream), "csa_indexer_loss");
}

size_t csa_indexer_loss_dense_workspace(const csa_dims* dm, size_t budget)
{
    if (!dm || dm->b < 1 || dm->sq < 1 || dm->ratio < 1) return 0;
    if (dm->idx_dim != 32 && dm->idx_dim != 64 && dm->idx_dim != 128) return 0;
    return csa::indexer_loss_dense_workspace_bytes(loss_args(dm), budget);
}

int csa_indexer_loss_dense(const csa_dims* dm, int dtype, const void* q, const void* c, const float* lse,
                           const void* q_i, const void* k_i, const float* w, float scale, const float* dkl,
                           float* kl, void* dq_i, float* dw, float* dk_i, void* ws, size_t ws_bytes, void* stream)
{
    const char* fn = "csa_indexer_loss_dense";
    int rc = check_common(dm, dtype, fn);
    if (rc) return rc;
    if ((rc = check_loss(dm, dtype, fn, true))) return rc;
    if (!std::isfinite(scale)) return fail(CSA_ERR_ARG, "%s: scale is not finite", fn);
    const bool blocks = dm->sq / dm->ratio > 0;
    if (!q || !lse || !q_i || !w || (blocks && (!c || !k_i)))
        return fail(CSA_ERR_ARG, "%s: q, c, lse, q_i, k_i and w must be non-NULL", fn);
    const bool any = dkl || dq_i || dw || dk_i;
    if (any && (!dkl || !dq_i || !dw || (blocks && !dk_i)))
        return fail(CSA_ERR_ARG, "%s: gradient gate: dkl, dq_i, dw and dk_i must all be given (or all be NULL)", fn);
    if ((rc = check_aligned(fn, {{"q", q}, {"c", c}, {"lse", lse}, {"q_i", q_i}, {"k_i", k_i}, {"w", w},
                                 {"dkl", dkl}, {"kl", kl}, {"dq_i", dq_i}, {"dw", dw}, {"dk_i", dk_i}})))
        return rc;
    if (!any && !kl) return ok();
    csa::LossArgs a = loss_args(dm);
    a.q = q; a.c = c; a.lse = lse; a.qi = q_i; a.ki = k_i; a.w = w;
    a.scale = scale; a.dkl = dkl; a.kl = kl; a.dqi = dq_i; a.dw = dw; a.dki = dk_i;
    const size_t need = csa::indexer_loss_dense_workspace_bytes(a, 0);
    if (!ws || ws_bytes < need)
        return fail(CSA_ERR_WORKSPACE, "%s: workspace of at least %zu bytes needed, %zu given", fn, need,
                    ws ? ws_bytes : (size_t)0);
    if (((uintptr_t)ws) & 15) return fail(CSA_ERR_ARG, "%s: workspace must be 16-byte aligned", fn);
    return hip_status(csa::indexer_loss_dense(a, dtype == CSA_BF16, (float*)ws, ws_bytes, (hipStream_t)stream), fn);
}

}  // extern "C"

namespace {

int check_gqa(const csa_gqa_dims* g, int dtype, const char* fn)
{
    if (!g) return fail(CSA_ERR_ARG, "%s: dims is NULL", fn);
    if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (g->b < 1 || g->sq < 1 || g->h < 1 || g->h_kv < 1 || g->d_qk < 1 || g->d_v < 1 || g->topk < 1)
        return fail(CSA_ERR_ARG, "%s: b, sq, h, h_kv, d_qk, d_v and topk must be >= 1", fn);
    if (g->h % g->h_kv) return fail(CSA_ERR_SHAPE, "%s: h=%d is not a multiple of h_kv=%d", fn, g->h, g->h_kv);
    if (g->h / g->h_kv > 64) return fail(CSA_ERR_UNSUPPORTED, "%s: %d query heads per group > 64", fn, g->h / g->h_kv);
    if (g->d_qk % 8 || g->d_v % 8) return fail(CSA_ERR_UNSUPPORTED, "%s: d_qk and d_v must be multiples of 8", fn);
    const int dp = g->d_qk + g->d_v;
    const bool ok = dtype == CSA_BF16 ? (dp == 64 || dp == 128 || dp == 256 || dp == 512) : (dp == 64 || dp == 128);
    if (!ok)
        return fail(CSA_ERR_UNSUPPORTED, "%s: d_qk + d_v = %d not in {64,128,256,512} (bf16) / {64,128} (fp32)", fn,
                    dp);
    if ((g->topk < g->sq ? g->topk : g->sq) > 2048) return fail(CSA_ERR_UNSUPPORTED, "%s: K' > 2048", fn);
    return CSA_OK;
}

csa::GqaArgs gqa_args(const csa_gqa_dims* g)
{
    csa::GqaArgs a{};
    a.b = g->b; a.S = g->sq; a.H = g->h; a.HKV = g->h_kv; a.DK = g->d_qk; a.DV = g->d_v;
    a.kp = g->topk < g->sq ? g->topk : g->sq;
    return a;
}

int check_ws(void* ws, size_t ws_bytes, size_t need, const char* fn)
{
    if (!ws || ws_bytes < need)
        return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : (size_t)0);
    if (((uintptr_t)ws) & 255) return fail(CSA_ERR_ARG, "%s: workspace must be 256-byte aligned", fn);
    return CSA_OK;
}

}  // namespace

extern "C" {

size_t csa_dsa_gqa_workspace(const csa_gqa_dims* g, int dtype, int backward)
{
    if (!g || g->b < 1 || g->sq < 1 || g->h < 1 || g->h_kv < 1 || g->h % g->h_kv || g->topk < 1) return 0;
    const csa::GqaArgs a = gqa_args(g);
    return csa::dsa_gqa_workspace_bytes(a, dtype == CSA_BF16, backward != 0);
}

int csa_dsa_gqa_fwd(const csa_gqa_dims* g, int dtype, const void* q, const void* k, const void* v,
                    const int32_t* idx, float scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_gqa(g, dtype, "csa_dsa_gqa_fwd");
    if (rc) return rc;
    if (!q || !k || !v || !idx || !out || !lse)
        return fail(CSA_ERR_ARG, "csa_dsa_gqa_fwd: q, k, v, idx, out and lse must be non-NULL");
    if (!std::isfinite(scale)) return fail(CSA_ERR_ARG, "csa_dsa_gqa_fwd: scale is not finite");
    csa::GqaArgs a = gqa_args(g);
    a.q = q; a.k = k; a.v = v; a.idx = idx; a.scale = scale; a.out = out; a.lse = lse;
    if ((rc = check_ws(ws, ws_bytes, csa::dsa_gqa_workspace_bytes(a, dtype == CSA_BF16, false), "csa_dsa_gqa_fwd")))
        return rc;
    return hip_status(csa::dsa_gqa_fwd(a, dtype == CSA_BF16, ws, (hipStream_t)stream), "csa_dsa_gqa_fwd");
}

int csa_dsa_gqa_bwd(const csa_gqa_dims* g, int dtype, const void* q, const void* k, const void* v,
                    const int32_t* idx, float scale, const void* out, const float* lse, const void* dout, void* dq,
                    float* dk, float* dv, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_gqa(g, dtype, "csa_dsa_gqa_bwd");
    if (rc) return rc;
    if (!q || !k || !v || !idx || !out || !lse || !dout)
        return fail(CSA_ERR_ARG, "csa_dsa_gqa_bwd: q, k, v, idx, out, lse and dout must be non-NULL");
    if (!dq || !dk || !dv)
        return fail(CSA_ERR_ARG, "csa_dsa_gqa_bwd: gradient gate: dq, dk and dv must all be given");
    if (!std::isfinite(scale)) return fail(CSA_ERR_ARG, "csa_dsa_gqa_bwd: scale is not finite");
    csa::GqaArgs a = gqa_args(g);
    a.q = q; a.k = k; a.v = v; a.idx = idx; a.scale = scale; a.out = const_cast<void*>(out);
    a.lse = const_cast<float*>(lse); a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
    if ((rc = check_ws(ws, ws_bytes, csa::dsa_gqa_workspace_bytes(a, dtype == CSA_BF16, true), "csa_dsa_gqa_bwd")))
        return rc;
    return hip_status(csa::dsa_gqa_bwd(a, dtype == CSA_BF16, ws, (hipStream_t)stream), "csa_dsa_gqa_bwd");
}

}  // extern "C"
