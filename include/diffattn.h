/*
 * diffattn.h — C ABI of libdiffattn, differential softmax attention on MI355X (gfx950).
 *
 * The operation (DIFF Transformer attention head):
 *
 *   O = ( softmax(Q1 K1^T * s) - lambda * softmax(Q2 K2^T * s) ) V,   s = 1/sqrt(d) by default,
 *
 * with Q1, Q2, K1, K2 of width d and V of width dv (2d in the DIFF V1 model), as defined in
 * "Differential Transformer: Noise-Canceling Attention by Subtraction", section "The mechanism",
 * and in "Differential Transformer: softmax can't say zero, so it subtracts", section
 * "The mechanism, exactly" (both maps are ordinary causal maps reading the same values).
 * The V1 epilogue is a per-head RMSNorm over the dv channels times an optional weight, then a
 * fixed multiply by (1 - lambda_init) ("softmax can't say zero", section "The row no longer sums
 * to one"). DIFF V2 pairs query heads 2p and 2p+1 of one GQA group, takes lambda per token and
 * pair, and drops the norm ("softmax can't say zero", section "DIFF V2: what the authors
 * changed"; "Differential Transformer V2").
 *
 * Conventions shared by every entry point:
 *  - Tensors are token-major: logical shape [batch, tokens, heads, dim]. A diffattn_tensor gives
 *    the base pointer and the batch / token / head strides IN ELEMENTS; the dim stride is 1.
 *    Any such strided view works (e.g. Q1 and Q2 as two halves of one packed [B,N,H,2,d] tensor).
 *  - Pointers passed to compute entry points are DEVICE pointers on the current HIP device,
 *    except where stated. bf16 tensors must be 16-byte aligned, and every stride a multiple of 8
 *    elements, for the bf16 MFMA kernels; other layouts are served by the generic kernel.
 *  - Output dtype equals input dtype. `out` must not alias any input.
 *  - Ownership: the caller owns every buffer, the workspace and the stream. The library allocates
 *    no device memory and keeps no state between calls except the thread-local error text.
 *  - Execution is asynchronous on `stream` (a hipStream_t; NULL = the default stream). Results are
 *    valid after the stream is synchronised. No entry point synchronises.
 *  - Errors: every argument is validated BEFORE any HIP call, so a non-OK return has launched
 *    nothing and written nothing. diffattn_last_error() returns a thread-local description of the
 *    last non-OK status. DIFFATTN_ERR_HIP reports a failed kernel launch.
 *  - All entry points are reentrant; calls on one stream execute in order.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIFFATTN_OK = 0,
    DIFFATTN_ERR_ARG = 1,          /* invalid argument: null pointer, bad size or stride */
    DIFFATTN_ERR_UNSUPPORTED = 2,  /* valid math that no kernel of the library serves */
    DIFFATTN_ERR_WORKSPACE = 3,    /* workspace smaller than diffattn_decode_workspace_size() */
    DIFFATTN_ERR_HIP = 4           /* a HIP call or kernel launch failed */
} diffattn_status;

typedef enum { DIFFATTN_F32 = 0, DIFFATTN_BF16 = 1 } diffattn_dtype;

typedef enum {
    DIFFATTN_EPI_NONE = 0,          /* O as defined above */
    DIFFATTN_EPI_RMSNORM_SCALE = 1  /* O <- O / sqrt(mean_c O_c^2 + eps) * w_c * (1 - lambda_init) */
} diffattn_epilogue;

/*
 * How a DIFF V2 entry point reads its lambda buffer. DIFF V2 learns lambda per token and per head
 * pair as the sigmoid of a linear projection of the token ("softmax can't say zero, so it
 * subtracts", section "DIFF V2: what the authors changed"; "Differential Transformer V2").
 */
typedef enum {
    DIFFATTN_LAMBDA_VALUE = 0,   /* lam holds lambda itself, used as given */
    DIFFATTN_LAMBDA_SIGMOID = 1  /* lam holds the projected logits z; the kernels use 1 / (1 + e^-z) */
} diffattn_lambda_mode;

/* A strided [batch, tokens, heads, dim] view; strides in elements, dim stride 1. */
typedef struct {
    void* ptr;
    int64_t s_batch;
    int64_t s_seq;
    int64_t s_head;
} diffattn_tensor;

/* Thread-local text for the last non-OK status returned on this thread ("" if none). */
const char* diffattn_last_error(void);

/* Library version, e.g. 100 for 0.1.0. */
int diffattn_version(void);

/*
 * lambda_init(l) = 0.8 - 0.6 * exp(-0.3 * (l - 1)), layer index l >= 1 (about 0.2 at l = 1,
 * tending to 0.8). "Noise-Canceling Attention by Subtraction", section "Making lambda learnable
 * and stable". Host function; returns NaN for layer < 1.
 */
double diffattn_lambda_init(int layer);

/*
 * lambda_out[r] = exp(lq1[r] . lk1[r]) - exp(lq2[r] . lk2[r]) + lambda_init(layer), r < n.
 * "Noise-Canceling Attention by Subtraction", section "Making lambda learnable and stable".
 *  lq1, lk1, lq2, lk2: DEVICE fp32 [n, dim] row-major (one row per head; n = 1 for one lambda
 *                      per layer). lambda_out: DEVICE fp32 [n].
 *  Dot products accumulate in fp32 and exp is evaluated in fp32.
 *  Errors: ERR_ARG if a pointer is NULL, n < 1, dim < 1 or layer < 1.
 */
diffattn_status diffattn_lambda(const float* lq1, const float* lk1, const float* lq2,
                                const float* lk2, int n, int dim, int layer, float* lambda_out,
                                void* stream);

/*
 * DIFF V1 forward (prefill), one output row per query token and head: the two softmax maps over the
 * same visible keys, their difference with lambda, times V ("Differential Transformer:
 * Noise-Canceling Attention by Subtraction", section "The mechanism"; "softmax can't say zero, so
 * it subtracts", section "The mechanism, exactly"), then optionally the per-head RMSNorm and the
 * (1 - lambda_init) multiply ("Noise-Canceling Attention by Subtraction", section "Making lambda
 * learnable and stable", items 1-2; "softmax can't say zero", section "The row no longer sums to
 * one").
 *  q1, q2: [batch, seq_q, heads, d];  k1, k2: [batch, seq_k, heads, d];  v: [batch, seq_k, heads, dv]
 *  out:    [batch, seq_q, heads, dv], same dtype as the inputs.
 *  lambda: DEVICE fp32 [heads] (per-layer lambda: pass equal entries). Any real value is accepted.
 *  causal: nonzero masks key j for query i unless j <= i + (seq_k - seq_q) (aligned to the last
 *          key; the ordinary j <= i when seq_q == seq_k). Masked keys drop out of both maps'
 *          normalisers. Requires seq_q <= seq_k so that every row sees at least one key.
 *  epi, norm_w, eps, lambda_init: the epilogue; norm_w is DEVICE fp32 [dv] or NULL for ones.
 *  scale:  softmax scale; <= 0 selects 1/sqrt(d).
 *  Kernels: bf16 with d = 64, dv = 128 and aligned strides runs the MFMA kernel (one pass over
 *  K/V tiles, two online softmax states, fused epilogue); every other case (fp32, or bf16 of
 *  another width, d <= 256 and dv <= 512) runs the generic kernel.
 *  Errors: ERR_ARG for NULL pointers, non-positive sizes, causal with seq_q > seq_k, or non-finite
 *  eps/lambda_init; ERR_UNSUPPORTED for d > 256 or dv > 512; ERR_HIP if the launch fails.
 */
diffattn_status diffattn_fwd(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                             diffattn_tensor k1, diffattn_tensor k2, diffattn_tensor v, int batch,
                             int heads, int seq_q, int seq_k, int d, int dv, const float* lambda,
                             float lambda_init, int causal, diffattn_epilogue epi,
                             const float* norm_w, float eps, float scale, diffattn_tensor out,
                             void* stream);

/*
 * DIFF V1 forward with lambda computed from its re-parameterisation in the same pass ("Noise-
 * Canceling Attention by Subtraction", section "Making lambda learnable and stable"): for head h,
 * lambda_h = exp(lq1[h] . lk1[h]) - exp(lq2[h] . lk2[h]) + lambda_init(layer), then diffattn_fwd
 * with lambda_init = lambda_init(layer) in the epilogue. The whole forward step is one kernel.
 *  lq1, lk1, lq2, lk2: DEVICE fp32 [heads, lam_dim] contiguous.  layer >= 1.
 *  lambda_out: DEVICE fp32 [heads], written with lambda (bit-identical to diffattn_lambda's
 *  output for the same vectors), as the backward pass needs it.
 *  Other arguments as in diffattn_fwd. The bf16 d = 64, dv = 128 MFMA kernel computes lambda in
 *  the kernel; other shapes run the lambda kernel, then the generic kernel.
 *  Errors: as diffattn_fwd, and ERR_ARG for null vectors or lambda_out, lam_dim < 1, layer < 1.
 */
diffattn_status diffattn_fwd_lambda(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                                    diffattn_tensor k1, diffattn_tensor k2, diffattn_tensor v,
                                    int batch, int heads, int seq_q, int seq_k, int d, int dv,
                                    const float* lq1, const float* lk1, const float* lq2,
                                    const float* lk2, int lam_dim, int layer, float* lambda_out,
                                    int causal, diffattn_epilogue epi, const float* norm_w,
                                    float eps, float scale, diffattn_tensor out, void* stream);

/*
 * Dynamic absmax quantisation of a score operand (Q1, Q2, K1 or K2) to fp8, OCP e4m3 (4 exponent
 * bits, bias 7, 3 mantissa bits, largest finite value 448), for diffattn_fwd_fp8. The pages report
 * DIFF's advantage for attention logits under dynamic absmax post-training quantisation
 * ("softmax can't say zero, so it subtracts", section "Outliers, and the low-bit claim"); the
 * granularity they leave open is taken here as one scale per (batch, head) slice:
 *   amax[b, h] = max |x[b, :, h, :]|,  scales[b, h] = amax / 448 (1 when amax = 0),
 *   out = e4m3 code of x * (448 / amax) (fp32 product; 1 when amax = 0), rounded to nearest
 *   even, so x is about out * scales[b, h].
 *  x: bf16 [batch, tokens, heads, dim] view, finite values; dim even.
 *  out: one-byte [batch, tokens, heads, dim] view (strides in bytes, even), written with the codes.
 *  scales, amax: DEVICE fp32 [batch, heads] contiguous, written.
 *  Kernels: one block per (batch, head) slice when there are at least 256 short slices (up to
 *  4096 x 128 elements), else per-block maxima merged by an atomic max on the fp32 bit pattern (exact, so the result
 *  does not depend on the order) and a conversion kernel; conversion by v_cvt_pk_fp8_f32.
 *  Errors: ERR_ARG (null pointers, sizes, odd dim or strides), ERR_HIP.
 */
diffattn_status diffattn_quantize_fp8(diffattn_tensor x, int batch, int tokens, int heads, int dim,
                                      diffattn_tensor out, float* scales, float* amax, void* stream);

/*
 * The four score operands of one fp8 forward quantised in one call: diffattn_quantize_fp8 of
 * q1, q2 (seq_q tokens) and k1, k2 (seq_k tokens), same arithmetic and bit-identical codes.
 *  q1, q2, k1, k2: bf16 views as in diffattn_quantize_fp8;  oq1, oq2, ok1, ok2: their code views.
 *  scales, amax: DEVICE fp32 [4, batch, heads] contiguous, operand order q1, q2, k1, k2 (so
 *  scales, scales + batch * heads, ... are the sq1, sq2, sk1, sk2 of diffattn_fwd_fp8).
 *  Kernels: one launch for all four when every slice fits in the registers of a 1024-thread block
 *  (tokens * dim <= 131072, 16-byte aligned views): each slice read once, its amax taken, its codes
 *  written; else diffattn_quantize_fp8's kernels operand by operand.
 *  Errors: as diffattn_quantize_fp8.
 */
diffattn_status diffattn_quantize_fp8_qk(diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                                         diffattn_tensor k2, int batch, int seq_q, int seq_k, int heads,
                                         int dim, diffattn_tensor oq1, diffattn_tensor oq2,
                                         diffattn_tensor ok1, diffattn_tensor ok2, float* scales,
                                         float* amax, void* stream);

/*
 * DIFF V1 forward with the attention logits taken on the fp8 matrix cores: S_k = Q_k K_k^T with
 * e4m3 operands (one v_mfma_f32_32x32x64_f8f6f4 per 32 x 32 tile and map), each product scaled
 * back by sq_k[b, h] * sk_k[b, h] in fp32; the softmaxes, the difference, the products with V
 * (bf16) and the epilogue as in diffattn_fwd.
 *  q1, q2: fp8 [batch, seq_q, heads, d];  k1, k2: fp8 [batch, seq_k, heads, d] (codes as written
 *  by diffattn_quantize_fp8; strides in bytes, multiples of 16, 16-byte aligned bases).
 *  sq1, sq2, sk1, sk2: DEVICE fp32 [batch, heads], the codes' scales.
 *  v, out, lambda, lambda_init, causal, epi, norm_w, eps, scale: as in diffattn_fwd (bf16).
 *  Serves d = 64, dv = 128 only. Errors: ERR_ARG, ERR_UNSUPPORTED (other d, dv, alignments),
 *  ERR_HIP.
 */
diffattn_status diffattn_fwd_fp8(diffattn_tensor q1, diffattn_tensor q2, diffattn_tensor k1,
                                 diffattn_tensor k2, const float* sq1, const float* sq2,
                                 const float* sk1, const float* sk2, diffattn_tensor v, int batch,
                                 int heads, int seq_q, int seq_k, int d, int dv, const float* lambda,
                                 float lambda_init, int causal, diffattn_epilogue epi,
                                 const float* norm_w, float eps, float scale, diffattn_tensor out,
                                 void* stream);

/*
 * Bytes of device workspace diffattn_decode needs for these sizes (0 on invalid sizes).
 * The workspace holds per-split partial results of both maps (running max, sum and a dv-wide
 * accumulator per map) in fp32.
 */
size_t diffattn_decode_workspace_size(int batch, int heads, int cache_len, int dv);

/*
 * DIFF V1 decode: one new query per (batch, head) against a KV cache; the query's own key and
 * value are expected to be in the cache already, so it attends to cache entries 0..len-1. The
 * operation is diffattn_fwd's for one query row over every cached key; the value cache is read
 * once for both maps ("Differential Transformer V2": unfused V1 decoding reads it twice).
 *  q1, q2: [batch, 1, heads, d] (the token stride is unused);
 *  k1c, k2c: [batch, cache_len, heads, d];  vc: [batch, cache_len, heads, dv]
 *  cache_lens: DEVICE int32 [batch] with 1 <= len <= cache_len, or NULL (every len = cache_len).
 *  lambda, lambda_init, epi, norm_w, eps, scale: as in diffattn_fwd.
 *  out: [batch, 1, heads, dv].
 *  workspace: DEVICE buffer of at least diffattn_decode_workspace_size(...) bytes, 256-byte
 *  aligned; its contents on entry do not matter.
 *  Kernels: bf16 with d = 64, dv = 128 runs a split-K kernel (each split streams its cache slice
 *  once with 16-byte loads, V read once for both maps) and a reduction kernel that merges the
 *  splits and applies the epilogue; the result does not depend on the split count's timing
 *  (fixed-order merge, no atomics). Other shapes run the generic kernel.
 *  Errors: ERR_ARG (NULL pointers, cache_len < 1, ...), ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP.
 *  A cache_lens entry outside 1..cache_len is clamped into that range on the device.
 */
diffattn_status diffattn_decode(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                                diffattn_tensor k1c, diffattn_tensor k2c, diffattn_tensor vc,
                                const int32_t* cache_lens, int batch, int heads, int cache_len,
                                int d, int dv, const float* lambda, float lambda_init,
                                diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                diffattn_tensor out, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * diffattn_decode without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops that keep allocation out of the step, and harnesses
 * that forbid hipMalloc. Same operation, arguments, kernels and results as diffattn_decode (the
 * outputs are bit-identical); the split partials go to a device array that the library holds,
 * one per GPU it runs on, created when the library's code is loaded on that GPU and kept until
 * the process ends. This call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.
 *  Limit: the sizes must need at most DIFFATTN_DECODE_NOALLOC_MAX_BYTES of workspace
 *  (diffattn_decode_workspace_size(batch, heads, cache_len, dv) <= 32 MiB, 1056 bytes per split
 *  of each (batch, head); that covers every batch * heads up to 31,775 at any cache length);
 *  larger sizes return ERR_WORKSPACE before any HIP call.
 *  stream: must belong to the current device (ERR_ARG otherwise); NULL is the current device's
 *  null stream.
 *  Concurrency: every call on one GPU uses that GPU's one array, so calls that overlap in time on
 *  one GPU (other streams, other threads) race on it and their results are undefined; calls on
 *  one stream are ordered and safe. Nothing in the array needs clearing between calls (every
 *  partial is written before it is read).
 *  Errors: as diffattn_decode, without ERR_WORKSPACE for a short workspace.
 */
#define DIFFATTN_DECODE_NOALLOC_MAX_BYTES (32u << 20)
diffattn_status diffattn_decode_noalloc(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                                        diffattn_tensor k1c, diffattn_tensor k2c, diffattn_tensor vc,
                                        const int32_t* cache_lens, int batch, int heads, int cache_len,
                                        int d, int dv, const float* lambda, float lambda_init,
                                        diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                                        diffattn_tensor out, void* stream);

/*
 * DIFF V1 decode against a paged KV cache: the same operation as diffattn_decode, with the cache
 * of each sequence held in fixed-size pages of shared pools, listed by a block table.
 *  k1_pages, k2_pages: [num_pages, page_size, heads, d];  v_pages: [num_pages, page_size, heads, dv]
 *     as strided views whose s_batch is the page stride (s_seq: token stride within a page).
 *  block_table: DEVICE int32 [batch, bt_stride]; token t of sequence b is row t % page_size of page
 *     block_table[b * bt_stride + t / page_size]. Entries for the pages of tokens 0..len_b-1 must be
 *     page indices below num_pages (an entry outside 0..num_pages-1 is clamped into it on the
 *     device); entries past them are not read.
 *  page_size: tokens per page, a positive multiple of 32 (a 32-token run of the kernels' tiles
 *     never straddles two pages).
 *  cache_lens: DEVICE int32 [batch] (each clamped into 1..max_len on the device), or NULL (every
 *     len = max_len).  max_len: the largest length; it sizes the split-K slices and the workspace
 *     (diffattn_decode_workspace_size(batch, heads, max_len, dv)), and bt_stride must hold
 *     ceil(max_len / page_size) entries.
 *  Other arguments as in diffattn_decode. Read traffic is the same as the contiguous decode's: each
 *  cached row once, plus one table entry per 32 tokens.
 *  Kernels: the split-K kernel of diffattn_decode, with a page lookup per 32-token run; bf16,
 *  d = 64, dv = 128 and 16-byte aligned views only.
 *  Errors: ERR_ARG (as diffattn_decode, and a null table, page_size not a multiple of 32, num_pages
 *  < 1, bt_stride too short), ERR_WORKSPACE, ERR_UNSUPPORTED (other dtypes, shapes or alignments),
 *  ERR_HIP.
 */
diffattn_status diffattn_decode_paged(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                                      diffattn_tensor k1_pages, diffattn_tensor k2_pages, diffattn_tensor v_pages,
                                      const int32_t* block_table, int64_t bt_stride, int num_pages, int page_size,
                                      const int32_t* cache_lens, int batch, int heads, int max_len, int d, int dv,
                                      const float* lambda, float lambda_init, diffattn_epilogue epi,
                                      const float* norm_w, float eps, float scale, diffattn_tensor out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * DIFF V2 forward: out[b, i, p] = O_{2p} - lam[b, i, p] * O_{2p+1}, where O_j is ordinary softmax
 * attention of query head j over KV head j / (2h / h_kv) (the heads of one GQA group are
 * contiguous, and a differenced pair sits in one group). No norm, no rescale ("softmax can't say
 * zero, so it subtracts", section "DIFF V2: what the authors changed"; "Differential Transformer
 * V2").
 *  q: [batch, seq, 2h, d];  k, v: [batch, seq, h_kv, d];  out: [batch, seq, h, d]
 *  lam: DEVICE fp32 [batch, seq, h] contiguous: lambda itself (lam_mode DIFFATTN_LAMBDA_VALUE) or
 *       the projected logits W_lambda x, whose sigmoid the kernel takes per row
 *       (DIFFATTN_LAMBDA_SIGMOID), so no separate pass over the logits is needed.
 *  causal: as in diffattn_fwd with seq_q = seq_k = seq.
 *  Requires 2h divisible by h_kv with an even group size (so no pair straddles two groups).
 *  Kernels: bf16 with d = 128 and aligned strides runs the MFMA kernel, in which one block owns a
 *  KV group and a query tile of all its query heads, so each K/V tile is read once per group;
 *  other cases run the generic kernel.
 *  Errors: ERR_ARG, ERR_UNSUPPORTED (d > 256), ERR_HIP.
 */
diffattn_status diffattn_v2_fwd(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k,
                                diffattn_tensor v, const float* lam, diffattn_lambda_mode lam_mode,
                                int batch, int seq, int h, int h_kv, int d, int causal, float scale,
                                diffattn_tensor out, void* stream);

/*
 * DIFF V1 training forward: diffattn_fwd plus what the backward pass needs.
 *  lse:  DEVICE fp32 [batch, heads, seq_q, 2], 8-byte aligned: per row and map the log-sum-exp of
 *        the scores in base 2, in units of scale * log2(e) * q.k (a weight is exp2(that - lse)).
 *  maps: DEVICE fp32 [batch, seq_q, heads, 2, dv], 16-byte aligned: A1 V and A2 V per row.
 *  The output and every other argument are those of diffattn_fwd.
 *  Serves bf16 with d = 64, dv = 128 and aligned strides (the MFMA kernel); ERR_UNSUPPORTED else.
 */
diffattn_status diffattn_fwd_train(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                                   diffattn_tensor k1, diffattn_tensor k2, diffattn_tensor v,
                                   int batch, int heads, int seq_q, int seq_k, int d, int dv,
                                   const float* lambda, float lambda_init, int causal,
                                   diffattn_epilogue epi, const float* norm_w, float eps,
                                   float scale, diffattn_tensor out, float* lse, float* maps,
                                   void* stream);

/* Bytes of device workspace diffattn_bwd needs (0 on invalid sizes): dL/do in bf16, two fp32
 * row statistics per row and per-block partial sums. */
size_t diffattn_bwd_workspace_size(int batch, int heads, int seq_q);

/*
 * DIFF V1 backward: the gradients of L = sum(dout * out) for the forward of diffattn_fwd_train
 * (same inputs and options), by the chain rule through "Noise-Canceling Attention by
 * Subtraction", sections "The mechanism" and "Making lambda learnable and stable": the RMSNorm *
 * (1 - lambda_init) epilogue, the difference of the two maps, the two softmaxes and the products.
 *  dout: [batch, seq_q, heads, dv];  lse, maps: the training forward's outputs for these inputs
 *  (maps 16-byte aligned, as diffattn_fwd_train requires).
 *  dq1, dq2: [batch, seq_q, heads, d];  dk1, dk2: [batch, seq_k, heads, d];  dv: like v; all
 *  written (bf16), fp32 accumulation inside.
 *  dlambda: DEVICE fp32 [heads] or NULL, written with dL/dlambda_h.  dnorm_w: DEVICE fp32 [dv] or
 *  NULL, written with dL/dw (only with the RMSNorm epilogue; summed over all heads and rows).
 *  workspace: DEVICE buffer of at least diffattn_bwd_workspace_size(...) bytes, 256-byte aligned.
 *  Kernels: a row pass (epilogue backward and the per-row dot products), a query-tile MFMA kernel
 *  for dQ, a key-tile MFMA kernel for dK and dV, and a fixed-order reduction; no atomics, so the
 *  result is bitwise reproducible. Serves bf16 with d = 64, dv = 128 and aligned strides.
 *  Errors: ERR_ARG, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP.
 */
diffattn_status diffattn_bwd(diffattn_dtype dtype, diffattn_tensor q1, diffattn_tensor q2,
                             diffattn_tensor k1, diffattn_tensor k2, diffattn_tensor v,
                             diffattn_tensor dout, int batch, int heads, int seq_q, int seq_k, int d,
                             int dv, const float* lambda, float lambda_init, int causal,
                             diffattn_epilogue epi, const float* norm_w, float eps, float scale,
                             const float* lse, const float* maps, diffattn_tensor dq1,
                             diffattn_tensor dq2, diffattn_tensor dk1, diffattn_tensor dk2,
                             diffattn_tensor dv_out, float* dlambda, float* dnorm_w,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradients of lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init with respect to the four
 * vectors, given dlambda per row ("Noise-Canceling Attention by Subtraction", section "Making
 * lambda learnable and stable"). All pointers DEVICE fp32; vectors [n, dim] row-major, dlambda [n].
 *  Errors: ERR_ARG if a pointer is NULL or n < 1 or dim < 1.
 */
diffattn_status diffattn_lambda_bwd(const float* lq1, const float* lk1, const float* lq2,
                                    const float* lk2, const float* dlambda, int n, int dim,
                                    float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                                    void* stream);

/*
 * DIFF V2 training forward: diffattn_v2_fwd plus what diffattn_v2_bwd needs.
 *  lse:  DEVICE fp32 [batch, h, seq, 2], 8-byte aligned: per row and pair the base-2 log-sum-exp
 *        of query heads 2p and 2p+1 (units of scale * log2(e) * q.k, as in diffattn_fwd_train).
 *  maps: DEVICE fp32 [batch, seq, h, 2, d], 16-byte aligned: A_{2p} V and A_{2p+1} V per row.
 *  The output and every other argument are those of diffattn_v2_fwd.
 *  Serves bf16 with d = 128, 1, 2, 4 or 8 pairs per KV head and aligned strides (the MFMA
 *  kernel); ERR_UNSUPPORTED else.
 */
diffattn_status diffattn_v2_fwd_train(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k,
                                      diffattn_tensor v, const float* lam, diffattn_lambda_mode lam_mode,
                                      int batch, int seq, int h, int h_kv, int d, int causal, float scale,
                                      diffattn_tensor out, float* lse, float* maps, void* stream);

/* Bytes of device workspace diffattn_v2_bwd needs (0 on invalid sizes): dout copied head-major
 * in bf16, two fp32 row statistics and lambda per row. */
size_t diffattn_v2_bwd_workspace_size(int batch, int h, int seq);

/*
 * DIFF V2 backward: the gradients of L = sum(dout * out) for the forward of diffattn_v2_fwd_train
 * (same inputs and options), by the chain rule through "softmax can't say zero, so it subtracts",
 * section "DIFF V2: what the authors changed" (out_p = A_{2p} V - lambda A_{2p+1} V with the
 * pair's GQA K and V, no norm): both softmaxes, the difference and the products.
 *  dout: [batch, seq, h, d];  lse, maps: the training forward's outputs for these inputs
 *  (maps 16-byte aligned, as diffattn_v2_fwd_train requires).
 *  dq: like q ([batch, seq, 2h, d]);  dk, dv: like k and v ([batch, seq, h_kv, d]), each summed
 *  over the query heads of its group; all written (bf16), fp32 accumulation inside.
 *  dlam: DEVICE fp32 [batch, seq, h], written with dL/dlam for what lam holds: dL/dlambda for
 *  DIFFATTN_LAMBDA_VALUE, dL/dz = dL/dlambda * lambda (1 - lambda) for DIFFATTN_LAMBDA_SIGMOID.
 *  workspace: DEVICE buffer of at least diffattn_v2_bwd_workspace_size(...) bytes, 256-byte
 *  aligned; its contents on entry do not matter.
 *  Kernels: a row pass (the per-row dot products and dlam), a query-tile MFMA kernel for dQ and a
 *  key-tile MFMA kernel for dK and dV that walks every pair of the KV head's group. No atomics:
 *  results are bitwise reproducible.
 *  Errors: ERR_ARG (null pointers, sizes, groups, lam_mode), ERR_WORKSPACE, ERR_UNSUPPORTED
 *  (other than bf16, d = 128, 1, 2, 4 or 8 pairs per KV head, aligned views), ERR_HIP.
 */
diffattn_status diffattn_v2_bwd(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k,
                                diffattn_tensor v, diffattn_tensor dout, const float* lam,
                                diffattn_lambda_mode lam_mode, int batch, int seq, int h, int h_kv, int d,
                                int causal, float scale, const float* lse, const float* maps,
                                diffattn_tensor dq, diffattn_tensor dk, diffattn_tensor dv, float* dlam,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace diffattn_v2_decode needs for these sizes (0 on invalid sizes). The
 * workspace holds, per cache slice and query head, the slice's shift, weight sum and 128-wide
 * accumulator in fp32. The slice count depends on how many blocks the current device holds at
 * once (its CU count), so query the size on the device that will run the decode.
 */
size_t diffattn_v2_decode_workspace_size(int batch, int h, int h_kv, int cache_len);

/*
 * DIFF V2 decode: the new token's 2h query heads against a GQA KV cache; output pair p is
 * O_{2p} - lam[b, p] * O_{2p+1}, where O_j is ordinary softmax attention of query head j over the
 * first len cache entries of KV head j / (2h / h_kv) ("softmax can't say zero", section "DIFF V2:
 * what the authors changed"; "Differential Transformer V2": decode reads the cache as ordinary GQA
 * attention does). The token's own key and value are expected to be in the cache already.
 *  q: [batch, 1, 2h, d] (the token stride is unused);  kc, vc: [batch, cache_len, h_kv, d]
 *  cache_lens: DEVICE int32 [batch] with 1 <= len <= cache_len, or NULL (every len = cache_len);
 *              an entry outside that range is clamped into it on the device.
 *  lam: DEVICE fp32 [batch, h] contiguous, lambda or its logits as lam_mode says (see
 *       diffattn_v2_fwd).   out: [batch, 1, h, d].
 *  scale: softmax scale; <= 0 selects 1/sqrt(d).
 *  workspace: DEVICE buffer of at least diffattn_v2_decode_workspace_size(...) bytes, 256-byte
 *  aligned; its contents on entry do not matter.
 *  Requires 2h divisible by h_kv with an even group size. Kernels: bf16 with d = 128, a group of
 *  2..32 query heads and aligned strides runs a split-K MFMA kernel that reads each cached K and V
 *  row once for the whole group, then a reduction that merges the slices in a fixed order (no
 *  atomics); other cases run the generic kernel.
 *  Errors: ERR_ARG, ERR_WORKSPACE, ERR_UNSUPPORTED (d > 256), ERR_HIP.
 */
diffattn_status diffattn_v2_decode(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor kc,
                                   diffattn_tensor vc, const int32_t* cache_lens, const float* lam,
                                   diffattn_lambda_mode lam_mode, int batch, int h, int h_kv,
                                   int cache_len, int d, float scale, diffattn_tensor out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * DIFF V2 decode against a paged KV cache: the same operation as diffattn_v2_decode, with the
 * cache of each sequence held in fixed-size pages of shared pools, listed by a block table.
 *  k_pages, v_pages: [num_pages, page_size, h_kv, d] as strided views whose s_batch is the page
 *     stride.  block_table, bt_stride, num_pages, page_size, cache_lens, max_len: as in
 *     diffattn_decode_paged (workspace: diffattn_v2_decode_workspace_size(batch, h, h_kv, max_len)).
 *  Other arguments as in diffattn_v2_decode.
 *  Kernels: the split-K MFMA kernel of diffattn_v2_decode, one table lookup per 32-key tile; bf16,
 *  d = 128, a group of 2..32 query heads and 16-byte aligned views only.
 *  Errors: ERR_ARG, ERR_WORKSPACE, ERR_UNSUPPORTED (other dtypes, shapes or alignments), ERR_HIP.
 */
diffattn_status diffattn_v2_decode_paged(diffattn_dtype dtype, diffattn_tensor q, diffattn_tensor k_pages,
                                         diffattn_tensor v_pages, const int32_t* block_table, int64_t bt_stride,
                                         int num_pages, int page_size, const int32_t* cache_lens, const float* lam,
                                         diffattn_lambda_mode lam_mode, int batch, int h, int h_kv, int max_len,
                                         int d, float scale, diffattn_tensor out, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Measurement helper, not part of the method: runs `blocks` blocks of 4 waves, each wave issuing
 * 8 x iters independent v_mfma_f32_32x32x16_bf16 (register operands only), so that the attainable
 * dense bf16 rate of the device can be timed beside the published peak. *flop (HOST) receives
 * the work of the launch. out: DEVICE fp32 [blocks * 256], written (keeps the work observable).
 * Errors: ERR_ARG (null pointers, blocks outside 1..2^20, iters < 1), ERR_HIP.
 */
diffattn_status diffattn_probe_mfma_peak(float* out, int blocks, int iters, double* flop, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
