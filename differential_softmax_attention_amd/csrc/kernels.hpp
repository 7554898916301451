// Kernel argument blocks and launchers (internal to libdiffattn; not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace diffattn {

// Generic kernel: one output row per wave. Head mapping for output head h:
//   query head of map 1 = h * q_hmul + q1_hoff, of map 2 = h * q_hmul + q2_hoff,
//   KV head = (h * q_hmul) / kv_hdiv.
// V1: q_hmul = 1, offsets 0, kv_hdiv = 1 (Q1/Q2 and K1/K2 are separate tensors).
// V2: q_hmul = 2, q1_hoff = 0, q2_hoff = 1, kv_hdiv = 2h / h_kv, K1 = K2 = K.
// lambda for (b, i, h) is lam[b * lams[0] + i * lams[1] + h * lams[2]].
struct GenericArgs {
    const void *q1, *q2, *k1, *k2, *v;
    void* out;
    int64_t q1s[3], q2s[3], k1s[3], k2s[3], vs[3], os[3];  // batch, token, head strides
    int q_hmul, q1_hoff, q2_hoff, kv_hdiv;
    const float* lam;
    int64_t lams[3];
    int lam_sigmoid;          // lam holds logits: lambda = sigmoid(lam)
    const int32_t* key_lens;  // per-batch key count (decode) or null
    int seq_q, seq_k, d, dv, causal, epi;
    const float* norm_w;
    float eps, lambda_init, scale;
};

hipError_t launch_generic(const GenericArgs& a, int batch, int heads, bool bf16_io, hipStream_t stream);

// MFMA forward kernels (bf16 in, fp32 accumulate, bf16 out).
// V1: separate Q1/Q2/K1/K2 tensors, d = 64, dv = 128, lambda per head, optional epilogue.
// V2: query heads 2p / 2p+1 of one tensor, shared K and V of the pair's KV head, d = dv = 128,
//     lambda per (b, token, pair), no epilogue.
struct MfmaFwdArgs {
    const void *q1, *q2, *k1, *k2, *v;
    void* out;
    int64_t q1s[3], q2s[3], k1s[3], k2s[3], vs[3], os[3];
    const float* lam;
    int64_t lams[3];
    int lam_sigmoid;  // V2: lam holds logits, lambda = sigmoid(lam)
    const float* norm_w;
    int batch, heads, seq_q, seq_k;
    int kv_group;     // V2: query heads per KV head (2h / h_kv); V1: unused
    int causal, epi;
    float eps, lambda_init, scale_log2;  // softmax scale * log2(e)
    // training outputs, both optional (null in inference): lse [batch, heads, seq_q, 2] holds each
    // map's log-sum-exp in base 2 of the scaled scores; maps [batch, seq_q, heads, 2, 128] holds
    // A1 V and A2 V in fp32 (V2: heads = pairs, the maps of query heads 2p and 2p+1)
    float* lse;
    float* maps;
    // fp8 score operands (launch_v1_fwd_fp8): Q1, Q2, K1, K2 hold OCP e4m3 codes (strides in bytes)
    // and these [batch, heads] factors turn the codes back into values
    const float *sq1, *sq2, *sk1, *sk2;
    // V1 lambda computed in the kernel (lq1 non-null): exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init
    // from the four [heads, lam_dim] vector sets, written to lam_out (optional)
    const float *lq1, *lk1, *lq2, *lk2;
    int lam_dim;
    float* lam_out;
};

hipError_t launch_v1_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream);
hipError_t launch_v2_fwd_mfma(const MfmaFwdArgs& a, hipStream_t stream);
hipError_t launch_v1_fwd_fp8(const MfmaFwdArgs& a, hipStream_t stream);
// the same kernels built under the max-ilp schedule, which the launches above use from kLongKeys keys
constexpr int kLongKeys = 4096;
hipError_t launch_v1_fwd_mfma_long(const MfmaFwdArgs& a, hipStream_t stream);
hipError_t launch_v2_fwd_mfma_long(const MfmaFwdArgs& a, hipStream_t stream);
hipError_t launch_v1_fwd_fp8_long(const MfmaFwdArgs& a, hipStream_t stream);

// Split-K decode (bf16, d = 64, dv = 128).
// Paged KV cache (block_table non-null): each cache tensor is a pool of pages whose batch stride
// is the page stride; token t of sequence b is row t % page_size of page
// block_table[b * bt_stride + t / page_size] (clamped into 0..num_pages-1). page_size is a
// multiple of 32, so a 32-token run that starts at a multiple of 32 lies in one page.
struct PagedCache {
    const int32_t* block_table;
    int64_t bt_stride;
    int page_size, num_pages;
    // page of token t of sequence b
    __device__ __forceinline__ int64_t page(int b, int t) const {
        const int p = block_table[(int64_t)b * bt_stride + t / page_size];
        return (int64_t)min(max(p, 0), num_pages - 1);
    }
};

struct DecodeArgs {
    const void *q1, *q2, *k1, *k2, *v;
    void* out;
    int64_t q1s[3], q2s[3], k1s[3], k2s[3], vs[3], os[3];
    const int32_t* cache_lens;
    const float* lam;
    const float* norm_w;
    float* ws;  // workspace: partials
    PagedCache pc;
    int batch, heads, cache_len, n_splits, split_len;
    int epi;
    float eps, lambda_init, scale_log2;
};

int decode_num_splits(int batch, int heads, int cache_len);
size_t decode_workspace_bytes(int batch, int heads, int cache_len, int dv);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Size of the device array that serves as diffattn_decode_noalloc's workspace, and its address
// on `device` (which must be the current device on the first call for it).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t decode_noalloc_scratch(int device, float** out);

// V2 split-K decode (bf16, d = 128, 2 <= group <= 32): q [batch, 1, 2h, d], caches
// [batch, L, h_kv, d], lambda [batch, h] at lam[b * lam_bs + p], out [batch, 1, h, d].
struct V2DecodeArgs {
    const void *q, *k, *v;
    void* out;
    int64_t qs[3], kcs[3], vcs[3], os[3];
    const int32_t* cache_lens;
    const float* lam;
    int64_t lam_bs;
    int lam_sigmoid;  // lam holds logits: lambda = sigmoid(lam)
    float* ws;  // workspace: per-slice partials
    PagedCache pc;
    int batch, h, h_kv, group, cache_len, n_splits, split_len;
    float scale_log2;
};

int v2_decode_num_splits(int batch, int h_kv, int group, int cache_len);
size_t v2_decode_workspace_bytes(int batch, int h, int h_kv, int cache_len);
bool v2_decode_group_ok(int group);
hipError_t launch_v2_decode(V2DecodeArgs a, hipStream_t stream);

// V1 backward (bf16, d = 64, dv = 128). Inputs as the forward plus dout [batch, seq_q, heads, 128]
// and the forward's training outputs; gradients in the inputs' layouts (bf16), dlam [heads] and
// dnorm_w [128] in fp32 (either may be null). go, dd, wpart, lampart live in the workspace.
struct BwdArgs {
    const void *q1, *q2, *k1, *k2, *v, *dout;
    int64_t q1s[3], q2s[3], k1s[3], k2s[3], vs[3], dos[3];
    void *dq1, *dq2, *dk1, *dk2, *dv;
    int64_t dq1s[3], dq2s[3], dk1s[3], dk2s[3], dvs[3];
    const float* lam;
    const float* norm_w;
    const float* lse;
    const float* maps;
    float* dlam;
    float* dnorm_w;
    bf16* go;        // [batch, heads, seq_q, 128] dL/do
    float* dd;       // [batch, heads, seq_q, 2] D1, D2
    float* wpart;    // [128][n_part] partial dL/dw
    float* lampart;  // [n_part] partial dlambda
    int n_part, pre_blocks;
    int batch, heads, seq_q, seq_k, causal, epi;
    float eps, lambda_init, scale_log2, scale;
};

size_t bwd_workspace_bytes(int batch, int heads, int seq_q);
hipError_t launch_bwd(BwdArgs a, void* workspace, hipStream_t stream);
hipError_t launch_lambda_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                             const float* dlam, int n, int dim, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                             hipStream_t stream);

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                         int n, int dim, float lambda_init, float* out, hipStream_t stream);

// DIFF V2 backward (bf16, d = 128): q [batch, seq, 2h, d], k, v [batch, seq, h_kv, d], dout
// [batch, seq, h, d]; lam [batch, seq, h] (values, or logits with lam_sigmoid); the training
// forward's lse [batch, h, seq, 2] and maps [batch, seq, h, 2, 128]; gradients dq, dk, dv like
// the inputs and dlam like lam.
struct V2BwdArgs {
    const void *q, *k, *v, *dout;
    int64_t qs[3], ks[3], vs[3], dos[3];
    void *dq, *dk, *dv;
    int64_t dqs[3], dks[3], dvs[3];
    const float* lam;
    int lam_sigmoid;
    const float* lse;
    const float* maps;
    float* dlam;
    // workspace: go [batch, h, seq, 128] bf16, dd [batch, h, seq, 2], lambda per row [batch, h, seq]
    bf16* go;
    float* dd;
    float* lamr;
    int batch, h, h_kv, group, seq, causal;
    float scale_log2, scale;
};

size_t v2_bwd_workspace_bytes(int batch, int h, int seq);
hipError_t launch_v2_bwd(V2BwdArgs a, void* workspace, hipStream_t stream);

// fp8 quantisation of a bf16 [batch, tokens, heads, dim] view (dim even): per (batch, head)
// amax = max |x|, scale s = amax / 448 (1 if amax = 0), out = OCP e4m3 codes of x / s.
struct Fp8QuantArgs {
    const void* x;
    void* out;
    int64_t xs[3], os[3];   // element strides (out: bytes)
    float* scales;          // [batch, heads], written
    float* amax;            // [batch, heads], written
    int batch, tokens, heads, dim;
};

hipError_t launch_quantize_fp8(const Fp8QuantArgs& a, hipStream_t stream);

// Up to four score operands quantised together (diffattn_quantize_fp8_qk): operand i has its own
// tensor, codes, token count, scales and amax; batch, heads and dim are shared.
struct Fp8QuantManyArgs {
    const void* x[4];
    void* out[4];
    int64_t xs[4][3], os[4][3];
    float* scales[4];
    float* amax[4];
    int tokens[4];
    int n, batch, heads, dim;
};
hipError_t launch_quantize_fp8_many(const Fp8QuantManyArgs& a, hipStream_t stream);

// Dense bf16 MFMA rate probe: `blocks` blocks of 4 waves, each wave 8 x iters MFMAs of 32x32x16
// (32768 flop each); out receives blocks * 256 floats.
hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t stream);

}  // namespace diffattn
