// C ABI of libdiffattn: argument validation (before any HIP call) and kernel dispatch.
// The operations and their argument conventions are documented in include/diffattn.h.
#include "../../include/diffattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

diffattn_status fail(diffattn_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

diffattn_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return DIFFATTN_OK;
    return fail(DIFFATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(diffattn_dtype dt) { return dt == DIFFATTN_BF16 ? 2 : 4; }

bool valid_dtype(diffattn_dtype dt) { return dt == DIFFATTN_F32 || dt == DIFFATTN_BF16; }

// Pointer non-null and aligned to its element size; strides non-negative.
diffattn_status check_tensor(const diffattn_tensor& t, const char* name, diffattn_dtype dt) {
    if (!t.ptr) return fail(DIFFATTN_ERR_ARG, "%s: null pointer", name);
    if (((uintptr_t)t.ptr) % elem_size(dt) != 0)
        return fail(DIFFATTN_ERR_ARG, "%s: pointer not aligned to its %zu-byte element", name, elem_size(dt));
    if (t.s_batch < 0 || t.s_seq < 0 || t.s_head < 0)
        return fail(DIFFATTN_ERR_ARG, "%s: negative stride", name);
    return DIFFATTN_OK;
}

// What the MFMA kernels read as 16-byte vectors: base 16-byte aligned, strides multiples of 8.
bool vec16_ok(const diffattn_tensor& t) {
    return ((uintptr_t)t.ptr) % 16 == 0 && t.s_batch % 8 == 0 && t.s_seq % 8 == 0 && t.s_head % 8 == 0;
}

void copy_strides(int64_t* dst, const diffattn_tensor& t) {
    dst[0] = t.s_batch;
    dst[1] = t.s_seq;
    dst[2] = t.s_head;
}

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / std::sqrt((float)d); }

}  // namespace

static diffattn_status fwd_impl(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                                diffattn_tensor k2, diffattn_tensor v, int batch, int heads, int seq_q, int seq_k,
                                int d, int dv, const float* lambda, float lambda_init, int causal,
                                diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                diffattn_tensor out, float* lse, float* maps, void* stream, const char* fn,
                                const float* const* lamvec = nullptr, int lam_dim = 0) {
    if (!valid_dtype(dtype)) return fail(DIFFATTN_ERR_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    const diffattn_tensor* ts[6] = {&q1, &q2, &k1, &k2, &v, &out};
    const char* names[6] = {"q1", "q2", "k1", "k2", "v", "out"};
    for (int i = 0; i < 6; ++i)
        if (diffattn_status s = check_tensor(*ts[i], names[i], dtype)) return s;
    if (!lambda) return fail(DIFFATTN_ERR_ARG, "%s: lambda is null", fn);
    if (batch < 1 || heads < 1 || seq_q < 1 || seq_k < 1 || d < 1 || dv < 1)
        return fail(DIFFATTN_ERR_ARG, "%s: sizes must be >= 1 (batch=%d heads=%d seq_q=%d seq_k=%d d=%d dv=%d)", fn,
                    batch, heads, seq_q, seq_k, d, dv);
    if (heads > 65535 || batch > 65535) return fail(DIFFATTN_ERR_ARG, "%s: batch and heads must be <= 65535", fn);
    if (causal && seq_q > seq_k)
        return fail(DIFFATTN_ERR_ARG, "%s: causal needs seq_q (%d) <= seq_k (%d)", fn, seq_q, seq_k);
    if (epi != DIFFATTN_EPI_NONE && epi != DIFFATTN_EPI_RMSNORM_SCALE)
        return fail(DIFFATTN_ERR_ARG, "%s: unknown epilogue %d", fn, (int)epi);
    if (epi == DIFFATTN_EPI_RMSNORM_SCALE && !(std::isfinite(eps) && eps >= 0.f && std::isfinite(lambda_init)))
        return fail(DIFFATTN_ERR_ARG, "%s: eps must be finite and >= 0, lambda_init finite", fn);
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "%s: scale must be finite", fn);
    if (d > 256 || dv > 512)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "%s: d=%d dv=%d exceed the supported d <= 256, dv <= 512", fn, d, dv);
    const float sc = resolve_scale(scale, d);
    hipStream_t st = (hipStream_t)stream;

    const bool mfma = dtype == DIFFATTN_BF16 && d == 64 && dv == 128 && vec16_ok(q1) && vec16_ok(q2) &&
                      vec16_ok(k1) && vec16_ok(k2) && vec16_ok(v) && vec16_ok(out);
    if (mfma) {
        diffattn::MfmaFwdArgs a{};
        a.q1 = q1.ptr; a.q2 = q2.ptr; a.k1 = k1.ptr; a.k2 = k2.ptr; a.v = v.ptr; a.out = out.ptr;
        copy_strides(a.q1s, q1); copy_strides(a.q2s, q2); copy_strides(a.k1s, k1); copy_strides(a.k2s, k2);
        copy_strides(a.vs, v); copy_strides(a.os, out);
        a.lam = lambda;
        a.lams[0] = 0; a.lams[1] = 0; a.lams[2] = 1;
        a.norm_w = norm_w;
        a.batch = batch; a.heads = heads; a.seq_q = seq_q; a.seq_k = seq_k;
        a.kv_group = 1;
        a.causal = causal ? 1 : 0;
        a.epi = epi == DIFFATTN_EPI_RMSNORM_SCALE;
        a.eps = eps; a.lambda_init = lambda_init;
        a.scale_log2 = sc * 1.4426950408889634f;
        a.lse = lse;
        a.maps = maps;
        if (lamvec) {
            // lambda from its vectors inside the kernel; `lambda` receives it
            a.lq1 = lamvec[0]; a.lk1 = lamvec[1]; a.lq2 = lamvec[2]; a.lk2 = lamvec[3];
            a.lam_dim = lam_dim;
            a.lam_out = const_cast<float*>(lambda);
        }
        return hip_status(diffattn::launch_v1_fwd_mfma(a, st), fn);
    }
    if (lamvec) {
        hipError_t e = diffattn::launch_lambda(lamvec[0], lamvec[1], lamvec[2], lamvec[3], heads, lam_dim, lambda_init,
                                               const_cast<float*>(lambda), st);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    diffattn::GenericArgs a{};
    a.q1 = q1.ptr; a.q2 = q2.ptr; a.k1 = k1.ptr; a.k2 = k2.ptr; a.v = v.ptr; a.out = out.ptr;
    copy_strides(a.q1s, q1); copy_strides(a.q2s, q2); copy_strides(a.k1s, k1); copy_strides(a.k2s, k2);
    copy_strides(a.vs, v); copy_strides(a.os, out);
    a.q_hmul = 1; a.q1_hoff = 0; a.q2_hoff = 0; a.kv_hdiv = 1;
    a.lam = lambda;
    a.lams[0] = 0; a.lams[1] = 0; a.lams[2] = 1;
    a.key_lens = nullptr;
    a.seq_q = seq_q; a.seq_k = seq_k; a.d = d; a.dv = dv;
    a.causal = causal ? 1 : 0;
    a.epi = epi == DIFFATTN_EPI_RMSNORM_SCALE;
    a.norm_w = norm_w; a.eps = eps; a.lambda_init = lambda_init; a.scale = sc;
    return hip_status(diffattn::launch_generic(a, batch, heads, dtype == DIFFATTN_BF16, st), fn);
}


extern "C" {

const char* diffattn_last_error(void) { return g_last_error.c_str(); }

int diffattn_version(void) { return 100; }

double diffattn_lambda_init(int layer) {
    if (layer < 1) return NAN;
    return 0.8 - 0.6 * std::exp(-0.3 * ((double)layer - 1.0));
}

diffattn_status diffattn_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int n,
                                int dim, int layer, float* lambda_out, void* stream) {
    if (!lq1 || !lk1 || !lq2 || !lk2 || !lambda_out) return fail(DIFFATTN_ERR_ARG, "diffattn_lambda: null pointer");
    if (n < 1 || dim < 1) return fail(DIFFATTN_ERR_ARG, "diffattn_lambda: n=%d dim=%d must be >= 1", n, dim);
    if (layer < 1) return fail(DIFFATTN_ERR_ARG, "diffattn_lambda: layer=%d must be >= 1", layer);
    const float li = (float)diffattn_lambda_init(layer);
    return hip_status(diffattn::launch_lambda(lq1, lk1, lq2, lk2, n, dim, li, lambda_out, (hipStream_t)stream),
                      "diffattn_lambda launch");
}

diffattn_status diffattn_fwd(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                             diffattn_tensor k2, diffattn_tensor v, int batch, int heads, int seq_q, int seq_k,
                             int d, int dv, const float* lambda, float lambda_init, int causal,
                             diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                             diffattn_tensor out, void* stream) {
    return fwd_impl(dtype, q1, q2, k1, k2, v, batch, heads, seq_q, seq_k, d, dv, lambda, lambda_init, causal, epi,
                    norm_w, eps, scale, out, nullptr, nullptr, stream, "diffattn_fwd");
}

diffattn_status diffattn_fwd_lambda(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                                    diffattn_tensor k2, diffattn_tensor v, int batch, int heads, int seq_q, int seq_k,
                                    int d, int dv, const float* lq1, const float* lk1, const float* lq2,
                                    const float* lk2, int lam_dim, int layer, float* lambda_out, int causal,
                                    diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                    diffattn_tensor out, void* stream) {
    if (!lq1 || !lk1 || !lq2 || !lk2 || !lambda_out)
        return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_lambda: lambda vectors and lambda_out must be non-null");
    if (lam_dim < 1) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_lambda: lam_dim=%d must be >= 1", lam_dim);
    if (layer < 1) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_lambda: layer=%d must be >= 1", layer);
    const float* vecs[4] = {lq1, lk1, lq2, lk2};
    return fwd_impl(dtype, q1, q2, k1, k2, v, batch, heads, seq_q, seq_k, d, dv, lambda_out,
                    (float)diffattn_lambda_init(layer), causal, epi, norm_w, eps, scale, out, nullptr, nullptr, stream,
                    "diffattn_fwd_lambda", vecs, lam_dim);
}

size_t diffattn_decode_workspace_size(int batch, int heads, int cache_len, int dv) {
    if (batch < 1 || heads < 1 || cache_len < 1 || dv < 1) return 0;
    return diffattn::decode_workspace_bytes(batch, heads, cache_len, dv);
}

// Page-table arguments: non-null table, page size a positive multiple of 32, a table row long
// enough for cache_len tokens.
static diffattn_status check_pages(const int32_t* block_table, int64_t bt_stride, int num_pages, int page_size,
                                   int cache_len, const char* fn) {
    if (!block_table) return fail(DIFFATTN_ERR_ARG, "%s: block_table is null", fn);
    if (page_size < 32 || page_size % 32 != 0)
        return fail(DIFFATTN_ERR_ARG, "%s: page_size=%d must be a positive multiple of 32", fn, page_size);
    if (num_pages < 1) return fail(DIFFATTN_ERR_ARG, "%s: num_pages=%d must be >= 1", fn, num_pages);
    if (cache_len >= 1 && bt_stride < (cache_len + page_size - 1) / page_size)
        return fail(DIFFATTN_ERR_ARG, "%s: bt_stride=%lld holds fewer than the %d pages of max_len=%d tokens", fn,
                    (long long)bt_stride, (cache_len + page_size - 1) / page_size, cache_len);
    return DIFFATTN_OK;
}

static diffattn_status decode_impl(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1c,
                                   diffattn_tensor k2c, diffattn_tensor vc, const int32_t* cache_lens, int batch,
                                   int heads, int cache_len, int d, int dv, const float* lambda, float lambda_init,
                                   diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                   diffattn_tensor out, void* workspace, size_t workspace_bytes, void* stream,
                                   const diffattn::PagedCache& pc, bool noalloc = false) {
    const char* fn_name = pc.block_table ? "diffattn_decode_paged" : noalloc ? "diffattn_decode_noalloc" : "diffattn_decode";
    if (!valid_dtype(dtype)) return fail(DIFFATTN_ERR_ARG, "diffattn_decode: unknown dtype %d", (int)dtype);
    const diffattn_tensor* ts[6] = {&q1, &q2, &k1c, &k2c, &vc, &out};
    const char* names[6] = {"q1", "q2", "k1c", "k2c", "vc", "out"};
    for (int i = 0; i < 6; ++i)
        if (diffattn_status s = check_tensor(*ts[i], names[i], dtype)) return s;
    if (!lambda) return fail(DIFFATTN_ERR_ARG, "diffattn_decode: lambda is null");
    if (batch < 1 || heads < 1 || cache_len < 1 || d < 1 || dv < 1)
        return fail(DIFFATTN_ERR_ARG, "diffattn_decode: sizes must be >= 1 (batch=%d heads=%d cache_len=%d d=%d dv=%d)",
                    batch, heads, cache_len, d, dv);
    if (heads > 65535 || batch > 65535) return fail(DIFFATTN_ERR_ARG, "diffattn_decode: batch and heads must be <= 65535");
    if (epi != DIFFATTN_EPI_NONE && epi != DIFFATTN_EPI_RMSNORM_SCALE)
        return fail(DIFFATTN_ERR_ARG, "diffattn_decode: unknown epilogue %d", (int)epi);
    if (epi == DIFFATTN_EPI_RMSNORM_SCALE && !(std::isfinite(eps) && eps >= 0.f && std::isfinite(lambda_init)))
        return fail(DIFFATTN_ERR_ARG, "diffattn_decode: eps must be finite and >= 0, lambda_init finite");
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "diffattn_decode: scale must be finite");
    if (d > 256 || dv > 512)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_decode: d=%d dv=%d exceed the supported d <= 256, dv <= 512", d, dv);
    const size_t need = diffattn_decode_workspace_size(batch, heads, cache_len, dv);
    if (noalloc) {
        if (need > diffattn::kNoallocScratchBytes)
            return fail(DIFFATTN_ERR_WORKSPACE,
                        "%s: these sizes need %zu bytes of workspace, more than the %zu bytes the library holds per "
                        "GPU; call diffattn_decode with a workspace instead", fn_name, need,
                        diffattn::kNoallocScratchBytes);
    } else {
        if (workspace_bytes < need)
            return fail(DIFFATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes < required %zu", fn_name, workspace_bytes,
                        need);
        if (need > 0 && (!workspace || ((uintptr_t)workspace) % 256 != 0))
            return fail(DIFFATTN_ERR_ARG, "%s: workspace must be non-null and 256-byte aligned", fn_name);
    }
    const float sc = resolve_scale(scale, d);
    hipStream_t st = (hipStream_t)stream;

    const bool split = dtype == DIFFATTN_BF16 && d == 64 && dv == 128 && vec16_ok(q1) && vec16_ok(q2) &&
                       vec16_ok(k1c) && vec16_ok(k2c) && vec16_ok(vc);
    if (pc.block_table && !split)
        return fail(DIFFATTN_ERR_UNSUPPORTED, "%s: a paged cache needs bf16, d=64, dv=128 and 16-byte aligned tensors",
                    fn_name);
    if (split) {
        diffattn::DecodeArgs a{};
        a.q1 = q1.ptr; a.q2 = q2.ptr; a.k1 = k1c.ptr; a.k2 = k2c.ptr; a.v = vc.ptr; a.out = out.ptr;
        copy_strides(a.q1s, q1); copy_strides(a.q2s, q2); copy_strides(a.k1s, k1c); copy_strides(a.k2s, k2c);
        copy_strides(a.vs, vc); copy_strides(a.os, out);
        a.cache_lens = cache_lens;
        a.pc = pc;
        a.lam = lambda;
        a.norm_w = norm_w;
        a.ws = (float*)workspace;
        if (noalloc) {
            // every argument is valid: the launch's device (the current one, which the stream must
            // belong to) and that device's copy of the library's scratch array
            int dev = 0;
            if (hipError_t e = hipGetDevice(&dev)) return hip_status(e, "diffattn_decode_noalloc: hipGetDevice");
            if (st) {
                hipDevice_t sdev = 0;
                if (hipError_t e = hipStreamGetDevice(st, &sdev))
                    return hip_status(e, "diffattn_decode_noalloc: hipStreamGetDevice");
                if ((int)sdev != dev)
                    return fail(DIFFATTN_ERR_ARG, "diffattn_decode_noalloc: the stream belongs to device %d but device "
                                "%d is current", (int)sdev, dev);
            }
            if (hipError_t e = diffattn::decode_noalloc_scratch(dev, &a.ws))
                return hip_status(e, "diffattn_decode_noalloc: scratch address");
        }
        a.batch = batch; a.heads = heads; a.cache_len = cache_len;
        a.epi = epi == DIFFATTN_EPI_RMSNORM_SCALE;
        a.eps = eps; a.lambda_init = lambda_init;
        a.scale_log2 = sc * 1.4426950408889634f;
        return hip_status(diffattn::launch_decode(a, st), "diffattn_decode launch");
    }
    diffattn::GenericArgs a{};
    a.q1 = q1.ptr; a.q2 = q2.ptr; a.k1 = k1c.ptr; a.k2 = k2c.ptr; a.v = vc.ptr; a.out = out.ptr;
    copy_strides(a.q1s, q1); copy_strides(a.q2s, q2); copy_strides(a.k1s, k1c); copy_strides(a.k2s, k2c);
    copy_strides(a.vs, vc); copy_strides(a.os, out);
    a.q_hmul = 1; a.q1_hoff = 0; a.q2_hoff = 0; a.kv_hdiv = 1;
    a.lam = lambda;
    a.lams[0] = 0; a.lams[1] = 0; a.lams[2] = 1;
    a.key_lens = cache_lens;
    a.seq_q = 1; a.seq_k = cache_len; a.d = d; a.dv = dv;
    a.causal = 0;
    a.epi = epi == DIFFATTN_EPI_RMSNORM_SCALE;
    a.norm_w = norm_w; a.eps = eps; a.lambda_init = lambda_init; a.scale = sc;
    return hip_status(diffattn::launch_generic(a, batch, heads, dtype == DIFFATTN_BF16, st), "diffattn_decode launch");
}

diffattn_status diffattn_decode(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1c,
                                diffattn_tensor k2c, diffattn_tensor vc, const int32_t* cache_lens, int batch,
                                int heads, int cache_len, int d, int dv, const float* lambda, float lambda_init,
                                diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                diffattn_tensor out, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(dtype, q1, q2, k1c, k2c, vc, cache_lens, batch, heads, cache_len, d, dv, lambda, lambda_init,
                       epi, norm_w, eps, scale, out, workspace, workspace_bytes, stream, diffattn::PagedCache{});
}

static_assert(DIFFATTN_DECODE_NOALLOC_MAX_BYTES == diffattn::kNoallocScratchBytes,
              "the header's limit is the size of the scratch array");

diffattn_status diffattn_decode_noalloc(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1c,
                                        diffattn_tensor k2c, diffattn_tensor vc, const int32_t* cache_lens, int batch,
                                        int heads, int cache_len, int d, int dv, const float* lambda,
                                        float lambda_init, diffattn_epilogue epi, const float* norm_w, float eps,
                                        float scale, diffattn_tensor out, void* stream) {
    return decode_impl(dtype, q1, q2, k1c, k2c, vc, cache_lens, batch, heads, cache_len, d, dv, lambda, lambda_init,
                       epi, norm_w, eps, scale, out, nullptr, 0, stream, diffattn::PagedCache{}, true);
}

diffattn_status diffattn_decode_paged(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                                      diffattn_tensor k1_pages, diffattn_tensor k2_pages, diffattn_tensor v_pages,
                                      const int32_t* block_table, int64_t bt_stride, int num_pages, int page_size,
                                      const int32_t* cache_lens, int batch, int heads, int max_len, int d, int dv,
                                      const float* lambda, float lambda_init, diffattn_epilogue epi,
                                      const float* norm_w, float eps, float scale, diffattn_tensor out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    if (diffattn_status s = check_pages(block_table, bt_stride, num_pages, page_size, max_len, "diffattn_decode_paged"))
        return s;
    diffattn::PagedCache pc{block_table, bt_stride, page_size, num_pages};
    return decode_impl(dtype, q1, q2, k1_pages, k2_pages, v_pages, cache_lens, batch, heads, max_len, d, dv, lambda,
                       lambda_init, epi, norm_w, eps, scale, out, workspace, workspace_bytes, stream, pc);
}

static bool valid_lam_mode(diffattn_lambda_mode m) { return m == DIFFATTN_LAMBDA_VALUE || m == DIFFATTN_LAMBDA_SIGMOID; }

// Conditions of the V2 MFMA kernels (forward, training forward, backward).
static bool v2_mfma_ok(diffattn_dtype dtype, int d, int group) {
    const int ppg = group / 2;
    return dtype == DIFFATTN_BF16 && d == 128 && (ppg == 1 || ppg == 2 || ppg == 4 || ppg == 8);
}

static diffattn_status v2_fwd_impl(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k, diffattn_tensor v,
                                   const float* lam, diffattn_lambda_mode lam_mode, int batch, int seq, int h,
                                   int h_kv, int d, int causal, float scale, diffattn_tensor out, float* lse,
                                   float* maps, void* stream) {
    if (!valid_dtype(dtype)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd: unknown dtype %d", (int)dtype);
    const diffattn_tensor* ts[4] = {&q, &k, &v, &out};
    const char* names[4] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i)
        if (diffattn_status s = check_tensor(*ts[i], names[i], dtype)) return s;
    if (!lam) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd: lam is null");
    if (!valid_lam_mode(lam_mode)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd: unknown lam_mode %d", (int)lam_mode);
    if (batch < 1 || seq < 1 || h < 1 || h_kv < 1 || d < 1)
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd: sizes must be >= 1 (batch=%d seq=%d h=%d h_kv=%d d=%d)", batch,
                    seq, h, h_kv, d);
    if (batch > 65535 || h > 65535) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd: batch and h must be <= 65535");
    if ((2 * h) % h_kv != 0 || ((2 * h) / h_kv) % 2 != 0)
        return fail(DIFFATTN_ERR_ARG,
                    "diffattn_v2_fwd: 2h=%d query heads must split into h_kv=%d groups of an even size (a pair may not "
                    "straddle two groups)", 2 * h, h_kv);
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd: scale must be finite");
    if (d > 256) return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_v2_fwd: d=%d exceeds the supported d <= 256", d);
    const float sc = resolve_scale(scale, d);
    hipStream_t st = (hipStream_t)stream;
    const int group = (2 * h) / h_kv;
    const int ppg = group / 2;

    const bool mfma = v2_mfma_ok(dtype, d, group) && vec16_ok(q) && vec16_ok(k) && vec16_ok(v) && vec16_ok(out);
    (void)ppg;
    if (lse && !mfma)
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_v2_fwd_train: serves bf16 with d = 128, 1, 2, 4 or 8 pairs per KV head and 16-byte "
                    "aligned tensors");
    if (mfma) {
        diffattn::MfmaFwdArgs a{};
        a.q1 = q.ptr; a.q2 = q.ptr; a.k1 = k.ptr; a.k2 = k.ptr; a.v = v.ptr; a.out = out.ptr;
        copy_strides(a.q1s, q); copy_strides(a.q2s, q); copy_strides(a.k1s, k); copy_strides(a.k2s, k);
        copy_strides(a.vs, v); copy_strides(a.os, out);
        a.lam = lam;
        a.lams[0] = (int64_t)seq * h; a.lams[1] = h; a.lams[2] = 1;
        a.lam_sigmoid = lam_mode == DIFFATTN_LAMBDA_SIGMOID;
        a.norm_w = nullptr;
        a.batch = batch; a.heads = h; a.seq_q = seq; a.seq_k = seq;
        a.kv_group = group;
        a.causal = causal ? 1 : 0;
        a.epi = 0;
        a.eps = 0.f; a.lambda_init = 0.f;
        a.scale_log2 = sc * 1.4426950408889634f;
        a.lse = lse;
        a.maps = maps;
        return hip_status(diffattn::launch_v2_fwd_mfma(a, st), "diffattn_v2_fwd launch");
    }
    diffattn::GenericArgs a{};
    a.q1 = q.ptr; a.q2 = q.ptr; a.k1 = k.ptr; a.k2 = k.ptr; a.v = v.ptr; a.out = out.ptr;
    copy_strides(a.q1s, q); copy_strides(a.q2s, q); copy_strides(a.k1s, k); copy_strides(a.k2s, k);
    copy_strides(a.vs, v); copy_strides(a.os, out);
    a.q_hmul = 2; a.q1_hoff = 0; a.q2_hoff = 1; a.kv_hdiv = group;
    a.lam = lam;
    a.lams[0] = (int64_t)seq * h; a.lams[1] = h; a.lams[2] = 1;
    a.lam_sigmoid = lam_mode == DIFFATTN_LAMBDA_SIGMOID;
    a.key_lens = nullptr;
    a.seq_q = seq; a.seq_k = seq; a.d = d; a.dv = d;
    a.causal = causal ? 1 : 0;
    a.epi = 0;
    a.norm_w = nullptr; a.eps = 0.f; a.lambda_init = 0.f; a.scale = sc;
    return hip_status(diffattn::launch_generic(a, batch, h, dtype == DIFFATTN_BF16, st), "diffattn_v2_fwd launch");
}

diffattn_status diffattn_v2_fwd(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k, diffattn_tensor v,
                                const float* lam, diffattn_lambda_mode lam_mode, int batch, int seq, int h, int h_kv,
                                int d, int causal, float scale, diffattn_tensor out, void* stream) {
    return v2_fwd_impl(dtype, q, k, v, lam, lam_mode, batch, seq, h, h_kv, d, causal, scale, out, nullptr, nullptr,
                       stream);
}

diffattn_status diffattn_v2_fwd_train(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k, diffattn_tensor v,
                                      const float* lam, diffattn_lambda_mode lam_mode, int batch, int seq, int h,
                                      int h_kv, int d, int causal, float scale, diffattn_tensor out, float* lse,
                                      float* maps, void* stream) {
    if (!lse || !maps) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd_train: lse and maps must be non-null");
    if (((uintptr_t)maps) % 16 != 0 || ((uintptr_t)lse) % 8 != 0)
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_fwd_train: maps must be 16-byte and lse 8-byte aligned");
    return v2_fwd_impl(dtype, q, k, v, lam, lam_mode, batch, seq, h, h_kv, d, causal, scale, out, lse, maps, stream);
}

size_t diffattn_v2_bwd_workspace_size(int batch, int h, int seq) {
    if (batch < 1 || h < 1 || seq < 1) return 0;
    return diffattn::v2_bwd_workspace_bytes(batch, h, seq);
}

diffattn_status diffattn_v2_bwd(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k, diffattn_tensor v,
                                diffattn_tensor dout, const float* lam, diffattn_lambda_mode lam_mode, int batch,
                                int seq, int h, int h_kv, int d, int causal, float scale, const float* lse,
                                const float* maps, diffattn_tensor dq, diffattn_tensor dk, diffattn_tensor dv,
                                float* dlam, void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_dtype(dtype)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: unknown dtype %d", (int)dtype);
    const diffattn_tensor* ts[7] = {&q, &k, &v, &dout, &dq, &dk, &dv};
    const char* names[7] = {"q", "k", "v", "dout", "dq", "dk", "dv"};
    for (int i = 0; i < 7; ++i)
        if (diffattn_status s = check_tensor(*ts[i], names[i], dtype)) return s;
    if (!lam || !lse || !maps || !dlam)
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: lam, lse, maps and dlam must be non-null");
    if (((uintptr_t)maps) % 16 != 0) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: maps must be 16-byte aligned");
    if (!valid_lam_mode(lam_mode)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: unknown lam_mode %d", (int)lam_mode);
    if (batch < 1 || seq < 1 || h < 1 || h_kv < 1 || d < 1)
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: sizes must be >= 1 (batch=%d seq=%d h=%d h_kv=%d d=%d)", batch,
                    seq, h, h_kv, d);
    if (batch > 65535 || h > 65535) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: batch and h must be <= 65535");
    if ((2 * h) % h_kv != 0 || ((2 * h) / h_kv) % 2 != 0)
        return fail(DIFFATTN_ERR_ARG,
                    "diffattn_v2_bwd: 2h=%d query heads must split into h_kv=%d groups of an even size", 2 * h, h_kv);
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: scale must be finite");
    const size_t need = diffattn_v2_bwd_workspace_size(batch, h, seq);
    if (workspace_bytes < need)
        return fail(DIFFATTN_ERR_WORKSPACE, "diffattn_v2_bwd: workspace of %zu bytes < required %zu", workspace_bytes,
                    need);
    if (!workspace || ((uintptr_t)workspace) % 256 != 0)
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_bwd: workspace must be non-null and 256-byte aligned");
    const int group = (2 * h) / h_kv;
    if (!v2_mfma_ok(dtype, d, group))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_v2_bwd: serves bf16 with d = 128 and 1, 2, 4 or 8 pairs per KV head");
    for (int i = 0; i < 7; ++i)
        if (!vec16_ok(*ts[i]))
            return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_v2_bwd: %s needs a 16-byte aligned base and strides that "
                        "are multiples of 8 elements", names[i]);
    diffattn::V2BwdArgs a{};
    a.q = q.ptr; a.k = k.ptr; a.v = v.ptr; a.dout = dout.ptr;
    copy_strides(a.qs, q); copy_strides(a.ks, k); copy_strides(a.vs, v); copy_strides(a.dos, dout);
    a.dq = dq.ptr; a.dk = dk.ptr; a.dv = dv.ptr;
    copy_strides(a.dqs, dq); copy_strides(a.dks, dk); copy_strides(a.dvs, dv);
    a.lam = lam;
    a.lam_sigmoid = lam_mode == DIFFATTN_LAMBDA_SIGMOID;
    a.lse = lse;
    a.maps = maps;
    a.dlam = dlam;
    a.batch = batch; a.h = h; a.h_kv = h_kv; a.group = group; a.seq = seq;
    a.causal = causal ? 1 : 0;
    const float sc = resolve_scale(scale, d);
    a.scale = sc;
    a.scale_log2 = sc * 1.4426950408889634f;
    return hip_status(diffattn::launch_v2_bwd(a, workspace, (hipStream_t)stream), "diffattn_v2_bwd launch");
}

size_t diffattn_v2_decode_workspace_size(int batch, int h, int h_kv, int cache_len) {
    if (batch < 1 || h < 1 || h_kv < 1 || cache_len < 1) return 0;
    if ((2 * h) % h_kv != 0) return 0;
    return diffattn::v2_decode_workspace_bytes(batch, h, h_kv, cache_len);
}

static diffattn_status v2_decode_impl(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor kc, diffattn_tensor vc,
                                      const int32_t* cache_lens, const float* lam, diffattn_lambda_mode lam_mode,
                                      int batch, int h, int h_kv,
                                      int cache_len, int d, float scale, diffattn_tensor out, void* workspace,
                                      size_t workspace_bytes, void* stream, const diffattn::PagedCache& pc) {
    if (!valid_dtype(dtype)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_decode: unknown dtype %d", (int)dtype);
    const diffattn_tensor* ts[4] = {&q, &kc, &vc, &out};
    const char* names[4] = {"q", "kc", "vc", "out"};
    for (int i = 0; i < 4; ++i)
        if (diffattn_status s = check_tensor(*ts[i], names[i], dtype)) return s;
    if (!lam) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_decode: lam is null");
    if (!valid_lam_mode(lam_mode))
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_decode: unknown lam_mode %d", (int)lam_mode);
    if (batch < 1 || h < 1 || h_kv < 1 || cache_len < 1 || d < 1)
        return fail(DIFFATTN_ERR_ARG,
                    "diffattn_v2_decode: sizes must be >= 1 (batch=%d h=%d h_kv=%d cache_len=%d d=%d)", batch, h,
                    h_kv, cache_len, d);
    if (batch > 65535 || h > 65535) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_decode: batch and h must be <= 65535");
    if ((2 * h) % h_kv != 0 || ((2 * h) / h_kv) % 2 != 0)
        return fail(DIFFATTN_ERR_ARG,
                    "diffattn_v2_decode: 2h=%d query heads must split into h_kv=%d groups of an even size (a pair may "
                    "not straddle two groups)", 2 * h, h_kv);
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "diffattn_v2_decode: scale must be finite");
    if (d > 256) return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_v2_decode: d=%d exceeds the supported d <= 256", d);
    const size_t need = diffattn_v2_decode_workspace_size(batch, h, h_kv, cache_len);
    if (workspace_bytes < need)
        return fail(DIFFATTN_ERR_WORKSPACE, "diffattn_v2_decode: workspace of %zu bytes < required %zu",
                    workspace_bytes, need);
    if (need > 0 && (!workspace || ((uintptr_t)workspace) % 256 != 0))
        return fail(DIFFATTN_ERR_ARG, "diffattn_v2_decode: workspace must be non-null and 256-byte aligned");
    const float sc = resolve_scale(scale, d);
    hipStream_t st = (hipStream_t)stream;
    const int group = (2 * h) / h_kv;

    const bool split = dtype == DIFFATTN_BF16 && d == 128 && diffattn::v2_decode_group_ok(group) && vec16_ok(q) &&
                       vec16_ok(kc) && vec16_ok(vc);
    if (pc.block_table && !split)
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_v2_decode_paged: a paged cache needs bf16, d=128, a group of 2..32 query heads and "
                    "16-byte aligned tensors");
    if (split) {
        diffattn::V2DecodeArgs a{};
        a.q = q.ptr; a.k = kc.ptr; a.v = vc.ptr; a.out = out.ptr;
        copy_strides(a.qs, q); copy_strides(a.kcs, kc); copy_strides(a.vcs, vc); copy_strides(a.os, out);
        a.cache_lens = cache_lens;
        a.pc = pc;
        a.lam = lam;
        a.lam_bs = h;
        a.lam_sigmoid = lam_mode == DIFFATTN_LAMBDA_SIGMOID;
        a.ws = (float*)workspace;
        a.batch = batch; a.h = h; a.h_kv = h_kv; a.group = group; a.cache_len = cache_len;
        a.scale_log2 = sc * 1.4426950408889634f;
        return hip_status(diffattn::launch_v2_decode(a, st), "diffattn_v2_decode launch");
    }
    diffattn::GenericArgs a{};
    a.q1 = q.ptr; a.q2 = q.ptr; a.k1 = kc.ptr; a.k2 = kc.ptr; a.v = vc.ptr; a.out = out.ptr;
    copy_strides(a.q1s, q); copy_strides(a.q2s, q); copy_strides(a.k1s, kc); copy_strides(a.k2s, kc);
    copy_strides(a.vs, vc); copy_strides(a.os, out);
    a.q_hmul = 2; a.q1_hoff = 0; a.q2_hoff = 1; a.kv_hdiv = group;
    a.lam = lam;
    a.lams[0] = h; a.lams[1] = 0; a.lams[2] = 1;
    a.lam_sigmoid = lam_mode == DIFFATTN_LAMBDA_SIGMOID;
    a.key_lens = cache_lens;
    a.seq_q = 1; a.seq_k = cache_len; a.d = d; a.dv = d;
    a.causal = 0;
    a.epi = 0;
    a.norm_w = nullptr; a.eps = 0.f; a.lambda_init = 0.f; a.scale = sc;
    return hip_status(diffattn::launch_generic(a, batch, h, dtype == DIFFATTN_BF16, st), "diffattn_v2_decode launch");
}

diffattn_status diffattn_v2_decode(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor kc, diffattn_tensor vc,
                                   const int32_t* cache_lens, const float* lam, diffattn_lambda_mode lam_mode,
                                   int batch, int h, int h_kv, int cache_len, int d, float scale, diffattn_tensor out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    return v2_decode_impl(dtype, q, kc, vc, cache_lens, lam, lam_mode, batch, h, h_kv, cache_len, d, scale, out,
                          workspace, workspace_bytes, stream, diffattn::PagedCache{});
}

diffattn_status diffattn_v2_decode_paged(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k_pages,
                                         diffattn_tensor v_pages, const int32_t* block_table, int64_t bt_stride,
                                         int num_pages, int page_size, const int32_t* cache_lens, const float* lam,
                                         diffattn_lambda_mode lam_mode, int batch, int h, int h_kv, int max_len, int d,
                                         float scale, diffattn_tensor out, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    if (diffattn_status s =
            check_pages(block_table, bt_stride, num_pages, page_size, max_len, "diffattn_v2_decode_paged"))
        return s;
    diffattn::PagedCache pc{block_table, bt_stride, page_size, num_pages};
    return v2_decode_impl(dtype, q, k_pages, v_pages, cache_lens, lam, lam_mode, batch, h, h_kv, max_len, d, scale,
                          out, workspace, workspace_bytes, stream, pc);
}

diffattn_status diffattn_fwd_train(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                                   diffattn_tensor k2, diffattn_tensor v, int batch, int heads, int seq_q, int seq_k,
                                   int d, int dv, const float* lambda, float lambda_init, int causal,
                                   diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                   diffattn_tensor out, float* lse, float* maps, void* stream) {
    if (!lse || !maps) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_train: lse and maps must be non-null");
    if (((uintptr_t)maps) % 16 != 0 || ((uintptr_t)lse) % 8 != 0)
        return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_train: maps must be 16-byte and lse 8-byte aligned");
    if (!(dtype == DIFFATTN_BF16 && d == 64 && dv == 128 && vec16_ok(q1) && vec16_ok(q2) && vec16_ok(k1) &&
          vec16_ok(k2) && vec16_ok(v) && vec16_ok(out)))
        return fail(DIFFATTN_ERR_UNSUPPORTED,
                    "diffattn_fwd_train: the training forward serves bf16 with d = 64, dv = 128 and aligned strides");
    return fwd_impl(dtype, q1, q2, k1, k2, v, batch, heads, seq_q, seq_k, d, dv, lambda, lambda_init, causal, epi,
                    norm_w, eps, scale, out, lse, maps, stream, "diffattn_fwd_train");
}

size_t diffattn_bwd_workspace_size(int batch, int heads, int seq_q) {
    if (batch < 1 || heads < 1 || seq_q < 1) return 0;
    return diffattn::bwd_workspace_bytes(batch, heads, seq_q);
}

diffattn_status diffattn_bwd(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                             diffattn_tensor k2, diffattn_tensor v, diffattn_tensor dout, int batch, int heads,
                             int seq_q, int seq_k, int d, int dv, const float* lambda, float lambda_init, int causal,
                             diffattn_epilogue epi, const float* norm_w, float eps, float scale, const float* lse,
                             const float* maps, diffattn_tensor dq1, diffattn_tensor dq2, diffattn_tensor dk1,
                             diffattn_tensor dk2, diffattn_tensor dv_out, float* dlambda, float* dnorm_w,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_dtype(dtype)) return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: unknown dtype %d", (int)dtype);
    const diffattn_tensor* ts[11] = {&q1, &q2, &k1, &k2, &v, &dout, &dq1, &dq2, &dk1, &dk2, &dv_out};
    const char* names[11] = {"q1", "q2", "k1", "k2", "v", "dout", "dq1", "dq2", "dk1", "dk2", "dv"};
    for (int i = 0; i < 11; ++i)
        if (diffattn_status s = check_tensor(*ts[i], names[i], dtype)) return s;
    if (!lambda || !lse || !maps) return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: lambda, lse and maps must be non-null");
    if (((uintptr_t)maps) % 16 != 0) return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: maps must be 16-byte aligned");
    if (batch < 1 || heads < 1 || seq_q < 1 || seq_k < 1 || d < 1 || dv < 1)
        return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: sizes must be >= 1 (batch=%d heads=%d seq_q=%d seq_k=%d d=%d dv=%d)",
                    batch, heads, seq_q, seq_k, d, dv);
    if (heads > 65535 || batch > 65535) return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: batch and heads must be <= 65535");
    if (causal && seq_q > seq_k)
        return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: causal needs seq_q (%d) <= seq_k (%d)", seq_q, seq_k);
    if (epi != DIFFATTN_EPI_NONE && epi != DIFFATTN_EPI_RMSNORM_SCALE)
        return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: unknown epilogue %d", (int)epi);
    if (epi == DIFFATTN_EPI_RMSNORM_SCALE && !(std::isfinite(eps) && eps >= 0.f && std::isfinite(lambda_init)))
        return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: eps must be finite and >= 0, lambda_init finite");
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: scale must be finite");
    const size_t need = diffattn_bwd_workspace_size(batch, heads, seq_q);
    if (workspace_bytes < need)
        return fail(DIFFATTN_ERR_WORKSPACE, "diffattn_bwd: workspace of %zu bytes < required %zu", workspace_bytes, need);
    if (!workspace || ((uintptr_t)workspace) % 256 != 0)
        return fail(DIFFATTN_ERR_ARG, "diffattn_bwd: workspace must be non-null and 256-byte aligned");
    if (!(dtype == DIFFATTN_BF16 && d == 64 && dv == 128))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_bwd: serves bf16 with d = 64, dv = 128");
    for (int i = 0; i < 11; ++i)
        if (!vec16_ok(*ts[i]))
            return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_bwd: %s needs a 16-byte aligned base and strides that are "
                        "multiples of 8 elements", names[i]);
    diffattn::BwdArgs a{};
    a.q1 = q1.ptr; a.q2 = q2.ptr; a.k1 = k1.ptr; a.k2 = k2.ptr; a.v = v.ptr; a.dout = dout.ptr;
    copy_strides(a.q1s, q1); copy_strides(a.q2s, q2); copy_strides(a.k1s, k1); copy_strides(a.k2s, k2);
    copy_strides(a.vs, v); copy_strides(a.dos, dout);
    a.dq1 = dq1.ptr; a.dq2 = dq2.ptr; a.dk1 = dk1.ptr; a.dk2 = dk2.ptr; a.dv = dv_out.ptr;
    copy_strides(a.dq1s, dq1); copy_strides(a.dq2s, dq2); copy_strides(a.dk1s, dk1); copy_strides(a.dk2s, dk2);
    copy_strides(a.dvs, dv_out);
    a.lam = lambda;
    a.norm_w = norm_w;
    a.lse = lse;
    a.maps = maps;
    a.dlam = dlambda;
    a.dnorm_w = epi == DIFFATTN_EPI_RMSNORM_SCALE ? dnorm_w : nullptr;
    a.batch = batch; a.heads = heads; a.seq_q = seq_q; a.seq_k = seq_k;
    a.causal = causal ? 1 : 0;
    a.epi = epi == DIFFATTN_EPI_RMSNORM_SCALE;
    a.eps = eps; a.lambda_init = lambda_init;
    const float sc = resolve_scale(scale, d);
    a.scale = sc;
    a.scale_log2 = sc * 1.4426950408889634f;
    return hip_status(diffattn::launch_bwd(a, workspace, (hipStream_t)stream), "diffattn_bwd launch");
}

// What the MFMA kernels read as 16-byte vectors of one-byte elements.
static bool vec16_bytes_ok(const diffattn_tensor& t) {
    return ((uintptr_t)t.ptr) % 16 == 0 && t.s_batch % 16 == 0 && t.s_seq % 16 == 0 && t.s_head % 16 == 0;
}

diffattn_status diffattn_quantize_fp8(diffattn_tensor x, int batch, int tokens, int heads, int dim,
                                      diffattn_tensor out, float* scales, float* amax, void* stream) {
    if (diffattn_status s = check_tensor(x, "x", DIFFATTN_BF16)) return s;
    if (!out.ptr) return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8: out is null");
    if (out.s_batch < 0 || out.s_seq < 0 || out.s_head < 0)
        return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8: negative stride in out");
    if (!scales || !amax) return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8: scales and amax must be non-null");
    if (batch < 1 || tokens < 1 || heads < 1 || dim < 2 || dim % 2 != 0)
        return fail(DIFFATTN_ERR_ARG,
                    "diffattn_quantize_fp8: sizes must be >= 1 and dim even (batch=%d tokens=%d heads=%d dim=%d)",
                    batch, tokens, heads, dim);
    if (batch > 65535 || heads > 65535)
        return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8: batch and heads must be <= 65535");
    if (((uintptr_t)out.ptr) % 2 != 0 || out.s_batch % 2 != 0 || out.s_seq % 2 != 0 || out.s_head % 2 != 0)
        return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8: out base and strides must be even (two codes per store)");
    diffattn::Fp8QuantArgs a{};
    a.x = x.ptr; a.out = out.ptr;
    copy_strides(a.xs, x); copy_strides(a.os, out);
    a.scales = scales; a.amax = amax;
    a.batch = batch; a.tokens = tokens; a.heads = heads; a.dim = dim;
    return hip_status(diffattn::launch_quantize_fp8(a, (hipStream_t)stream), "diffattn_quantize_fp8 launch");
}

diffattn_status diffattn_quantize_fp8_qk(diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1, diffattn_tensor k2,
                                         int batch, int seq_q, int seq_k, int heads, int dim, diffattn_tensor oq1,
                                         diffattn_tensor oq2, diffattn_tensor ok1, diffattn_tensor ok2, float* scales,
                                         float* amax, void* stream) {
    const diffattn_tensor* xs[4] = {&q1, &q2, &k1, &k2};
    const diffattn_tensor* os[4] = {&oq1, &oq2, &ok1, &ok2};
    const char* xn[4] = {"q1", "q2", "k1", "k2"};
    const char* on[4] = {"oq1", "oq2", "ok1", "ok2"};
    for (int i = 0; i < 4; ++i) {
        if (diffattn_status st = check_tensor(*xs[i], xn[i], DIFFATTN_BF16)) return st;
        if (!os[i]->ptr) return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8_qk: %s is null", on[i]);
        if (os[i]->s_batch < 0 || os[i]->s_seq < 0 || os[i]->s_head < 0)
            return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8_qk: negative stride in %s", on[i]);
        if (((uintptr_t)os[i]->ptr) % 2 != 0 || os[i]->s_batch % 2 != 0 || os[i]->s_seq % 2 != 0 ||
            os[i]->s_head % 2 != 0)
            return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8_qk: %s base and strides must be even", on[i]);
    }
    if (!scales || !amax) return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8_qk: scales and amax must be non-null");
    if (batch < 1 || seq_q < 1 || seq_k < 1 || heads < 1 || dim < 2 || dim % 2 != 0)
        return fail(DIFFATTN_ERR_ARG,
                    "diffattn_quantize_fp8_qk: sizes must be >= 1 and dim even (batch=%d seq_q=%d seq_k=%d heads=%d dim=%d)",
                    batch, seq_q, seq_k, heads, dim);
    if (batch > 65535 || heads > 65535)
        return fail(DIFFATTN_ERR_ARG, "diffattn_quantize_fp8_qk: batch and heads must be <= 65535");
    diffattn::Fp8QuantManyArgs a{};
    const int64_t bh = (int64_t)batch * heads;
    for (int i = 0; i < 4; ++i) {
        a.x[i] = xs[i]->ptr;
        a.out[i] = os[i]->ptr;
        copy_strides(a.xs[i], *xs[i]);
        copy_strides(a.os[i], *os[i]);
        a.scales[i] = scales + i * bh;
        a.amax[i] = amax + i * bh;
        a.tokens[i] = i < 2 ? seq_q : seq_k;
    }
    a.n = 4;
    a.batch = batch; a.heads = heads; a.dim = dim;
    return hip_status(diffattn::launch_quantize_fp8_many(a, (hipStream_t)stream), "diffattn_quantize_fp8_qk launch");
}

diffattn_status diffattn_fwd_fp8(diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1, diffattn_tensor k2,
                                 const float* sq1, const float* sq2, const float* sk1, const float* sk2,
                                 diffattn_tensor v, int batch, int heads, int seq_q, int seq_k, int d, int dv,
                                 const float* lambda, float lambda_init, int causal, diffattn_epilogue epi,
                                 const float* norm_w, float eps, float scale, diffattn_tensor out, void* stream) {
    const diffattn_tensor* f8[4] = {&q1, &q2, &k1, &k2};
    const char* f8n[4] = {"q1", "q2", "k1", "k2"};
    for (int i = 0; i < 4; ++i) {
        if (!f8[i]->ptr) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: %s is null", f8n[i]);
        if (f8[i]->s_batch < 0 || f8[i]->s_seq < 0 || f8[i]->s_head < 0)
            return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: negative stride in %s", f8n[i]);
    }
    if (diffattn_status s = check_tensor(v, "v", DIFFATTN_BF16)) return s;
    if (diffattn_status s = check_tensor(out, "out", DIFFATTN_BF16)) return s;
    if (!sq1 || !sq2 || !sk1 || !sk2) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: scale arrays must be non-null");
    if (!lambda) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: lambda is null");
    if (batch < 1 || heads < 1 || seq_q < 1 || seq_k < 1 || d < 1 || dv < 1)
        return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: sizes must be >= 1 (batch=%d heads=%d seq_q=%d seq_k=%d d=%d dv=%d)",
                    batch, heads, seq_q, seq_k, d, dv);
    if (heads > 65535 || batch > 65535) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: batch and heads must be <= 65535");
    if (causal && seq_q > seq_k)
        return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: causal needs seq_q (%d) <= seq_k (%d)", seq_q, seq_k);
    if (epi != DIFFATTN_EPI_NONE && epi != DIFFATTN_EPI_RMSNORM_SCALE)
        return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: unknown epilogue %d", (int)epi);
    if (epi == DIFFATTN_EPI_RMSNORM_SCALE && !(std::isfinite(eps) && eps >= 0.f && std::isfinite(lambda_init)))
        return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: eps must be finite and >= 0, lambda_init finite");
    if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_ARG, "diffattn_fwd_fp8: scale must be finite");
    if (d != 64 || dv != 128) return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_fwd_fp8: serves d = 64, dv = 128");
    for (int i = 0; i < 4; ++i)
        if (!vec16_bytes_ok(*f8[i]))
            return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_fwd_fp8: %s needs a 16-byte aligned base and strides that "
                        "are multiples of 16", f8n[i]);
    if (!vec16_ok(v) || !vec16_ok(out))
        return fail(DIFFATTN_ERR_UNSUPPORTED, "diffattn_fwd_fp8: v and out need 16-byte alignment and strides that are "
                    "multiples of 8 elements");
    diffattn::MfmaFwdArgs a{};
    a.q1 = q1.ptr; a.q2 = q2.ptr; a.k1 = k1.ptr; a.k2 = k2.ptr; a.v = v.ptr; a.out = out.ptr;
    copy_strides(a.q1s, q1); copy_strides(a.q2s, q2); copy_strides(a.k1s, k1); copy_strides(a.k2s, k2);
    copy_strides(a.vs, v); copy_strides(a.os, out);
    a.lam = lambda;
    a.norm_w = norm_w;
    a.batch = batch; a.heads = heads; a.seq_q = seq_q; a.seq_k = seq_k;
    a.causal = causal ? 1 : 0;
    a.epi = epi == DIFFATTN_EPI_RMSNORM_SCALE;
    a.eps = eps; a.lambda_init = lambda_init;
    a.scale_log2 = resolve_scale(scale, d) * 1.4426950408889634f;
    a.sq1 = sq1; a.sq2 = sq2; a.sk1 = sk1; a.sk2 = sk2;
    return hip_status(diffattn::launch_v1_fwd_fp8(a, (hipStream_t)stream), "diffattn_fwd_fp8 launch");
}

diffattn_status diffattn_probe_mfma_peak(float* out, int blocks, int iters, double* flop, void* stream) {
    if (!out || !flop) return fail(DIFFATTN_ERR_ARG, "diffattn_probe_mfma_peak: out and flop must be non-null");
    if (blocks < 1 || iters < 1 || blocks > (1 << 20))
        return fail(DIFFATTN_ERR_ARG, "diffattn_probe_mfma_peak: blocks=%d iters=%d out of range", blocks, iters);
    *flop = (double)blocks * 4 * 8 * (double)iters * 32768.0;
    return hip_status(diffattn::launch_mfma_peak(out, blocks, iters, (hipStream_t)stream),
                      "diffattn_probe_mfma_peak launch");
}

diffattn_status diffattn_lambda_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                                    const float* dlambda, int n, int dim, float* dlq1, float* dlk1, float* dlq2,
                                    float* dlk2, void* stream) {
    if (!lq1 || !lk1 || !lq2 || !lk2 || !dlambda || !dlq1 || !dlk1 || !dlq2 || !dlk2)
        return fail(DIFFATTN_ERR_ARG, "diffattn_lambda_bwd: null pointer");
    if (n < 1 || dim < 1) return fail(DIFFATTN_ERR_ARG, "diffattn_lambda_bwd: n=%d dim=%d must be >= 1", n, dim);
    return hip_status(diffattn::launch_lambda_bwd(lq1, lk1, lq2, lk2, dlambda, n, dim, dlq1, dlk1, dlq2, dlk2,
                                                  (hipStream_t)stream),
                      "diffattn_lambda_bwd launch");
}

}  // extern "C"
