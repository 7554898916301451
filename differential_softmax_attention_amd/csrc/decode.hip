// Differential-attention decode (one query per batch entry and head against a KV cache), bf16
// cache, d = 64, dv = 128, fp32 arithmetic.
//
// Decode is bound by reading the cache: per cached token K1 (128 B), K2 (128 B) and V (256 B).
// With two separate attention calls the V cache would be read twice ("Differential Transformer
// V2": V1 decoding loads the value cache twice with unfused kernels); here both maps consume each
// V row in the same pass, so every cache byte is read exactly once.
//
// Split-K: the cache of each (batch, head) is cut into n_splits slices. diffattn_decode_split
// streams one slice per 256-thread block: eight lanes own one cached token (16-byte loads: lane g
// reads K1/K2 channels 8g..8g+7 and V channels 16g..16g+15), the two scores are reduced over the
// eight lanes, and each lane group keeps its own online-softmax state (max, sum, 16 output
// channels per map). At the end of the slice the groups and waves are merged in a fixed order and
// the slice's partial (max, sum, 128-wide accumulator per map) is written to the workspace.
// diffattn_decode_reduce merges the partials of all slices in split order (log-sum-exp
// rescaling), forms O1/l1 - lambda O2/l2 and applies the RMSNorm * w * (1 - lambda_init)
// epilogue ("Noise-Canceling Attention by Subtraction", section "Making lambda learnable and
// stable"). No atomics: the result is bitwise reproducible.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

constexpr int kDV = 128;
constexpr int kPartial = 4 + 2 * kDV + 4;   // m1, l1, m2, l2, o1[128], o2[128], pad -> 264 floats
constexpr int kSplitThreads = 256;
constexpr int kUnroll = 4;                  // tokens per lane group per iteration
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kSplitThreads) void decode_split_kernel(DecodeArgs a) {
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane & 7;       // channel slot within the token's lane group
    const int kg = lane >> 3;     // token slot within the wave (0..7)

    int len = a.cache_len;
    if (a.cache_lens) len = min(max(a.cache_lens[b], 1), a.cache_len);
    const int ks = split * a.split_len;
    const int ke = min(ks + a.split_len, len);

    // query fragments (channels 8g..8g+7), pre-scaled by scale * log2(e)
    float q1[8], q2[8];
    {
        const u32x4 w1 = *(const u32x4*)((const bf16*)a.q1 + b * a.q1s[0] + (int64_t)h * a.q1s[2] + 8 * g);
        const u32x4 w2 = *(const u32x4*)((const bf16*)a.q2 + b * a.q2s[0] + (int64_t)h * a.q2s[2] + 8 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            q1[2 * j] = bf_lo(w1[j]) * a.scale_log2;
            q1[2 * j + 1] = bf_hi(w1[j]) * a.scale_log2;
            q2[2 * j] = bf_lo(w2[j]) * a.scale_log2;
            q2[2 * j + 1] = bf_hi(w2[j]) * a.scale_log2;
        }
    }
    // contiguous cache: batch b's rows; paged: the pool (the batch stride is the page stride)
    const bool paged = a.pc.block_table != nullptr;
    const int64_t bsel = paged ? 0 : b;
    const bf16* k1b = (const bf16*)a.k1 + bsel * a.k1s[0] + (int64_t)h * a.k1s[2] + 8 * g;
    const bf16* k2b = (const bf16*)a.k2 + bsel * a.k2s[0] + (int64_t)h * a.k2s[2] + 8 * g;
    const bf16* vb = (const bf16*)a.v + bsel * a.vs[0] + (int64_t)h * a.vs[2] + 16 * g;

    const int x1 = (lane ^ 1) << 2, x2 = (lane ^ 2) << 2, x4 = (lane ^ 4) << 2;

    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    float o1[16], o2[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) { o1[c] = 0.f; o2[c] = 0.f; }

    constexpr int kStep = 4 * 8 * kUnroll;   // tokens per block iteration
    for (int t0 = ks; t0 < ke; t0 += kStep) {
        u32x4 rk1[kUnroll], rk2[kUnroll], rv0[kUnroll], rv1[kUnroll];
        bool valid[kUnroll];
        // this wave's 32 tokens start at tw (a multiple of 32, so they share one page); tokens
        // past the slice end load row tb instead (a valid row of the same page) and are dropped
        const int tw = t0 + wave * 8 * kUnroll;
        const int tb = tw < ke ? tw : ks;
        const bf16 *k1w, *k2w, *vw;   // row of token tb
        if (paged) {
            const int64_t pg = a.pc.page(b, tb), in = tb % a.pc.page_size;
            k1w = k1b + pg * a.k1s[0] + in * a.k1s[1];
            k2w = k2b + pg * a.k2s[0] + in * a.k2s[1];
            vw = vb + pg * a.vs[0] + in * a.vs[1];
        } else {
            k1w = k1b + (int64_t)tb * a.k1s[1];
            k2w = k2b + (int64_t)tb * a.k2s[1];
            vw = vb + (int64_t)tb * a.vs[1];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int t = tw + u * 8 + kg;
            valid[u] = t < ke;
            const int64_t dt = valid[u] ? t - tb : 0;
            rk1[u] = *(const u32x4*)(k1w + dt * a.k1s[1]);
            rk2[u] = *(const u32x4*)(k2w + dt * a.k2s[1]);
            const bf16* vr = vw + dt * a.vs[1];
            rv0[u] = *(const u32x4*)(vr);
            rv1[u] = *(const u32x4*)(vr + 8);
        }
        float s1[kUnroll], s2[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float d1 = 0.f, d2 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                d1 = fmaf(q1[2 * j], bf_lo(rk1[u][j]), d1);
                d1 = fmaf(q1[2 * j + 1], bf_hi(rk1[u][j]), d1);
                d2 = fmaf(q2[2 * j], bf_lo(rk2[u][j]), d2);
                d2 = fmaf(q2[2 * j + 1], bf_hi(rk2[u][j]), d2);
            }
            d1 += lane_xor(d1, x1);
            d2 += lane_xor(d2, x1);
            d1 += lane_xor(d1, x2);
            d2 += lane_xor(d2, x2);
            d1 += lane_xor(d1, x4);
            d2 += lane_xor(d2, x4);
            s1[u] = valid[u] ? d1 : -INFINITY;   // already in log2 units
            s2[u] = valid[u] ? d2 : -INFINITY;
        }
        float mx1 = s1[0], mx2 = s2[0];
#pragma unroll
        for (int u = 1; u < kUnroll; ++u) { mx1 = fmaxf(mx1, s1[u]); mx2 = fmaxf(mx2, s2[u]); }
        const bool need = (mx1 > m1 + kRescaleThreshold) || (mx2 > m2 + kRescaleThreshold);
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mn1 = fmaxf(m1, mx1), mn2 = fmaxf(m2, mx2);
            // a group with no valid token yet keeps m = -inf; guard exp2(-inf - -inf)
            const float al1 = (mn1 == -INFINITY) ? 1.f : fast_exp2(m1 - mn1);
            const float al2 = (mn2 == -INFINITY) ? 1.f : fast_exp2(m2 - mn2);
            m1 = mn1;
            m2 = mn2;
            l1 *= al1;
            l2 *= al2;
#pragma unroll
            for (int c = 0; c < 16; ++c) { o1[c] *= al1; o2[c] *= al2; }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float p1 = valid[u] ? fast_exp2(s1[u] - m1) : 0.f;
            const float p2 = valid[u] ? fast_exp2(s2[u] - m2) : 0.f;
            l1 += p1;
            l2 += p2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float va = bf_lo(rv0[u][j]), vb2 = bf_hi(rv0[u][j]);
                const float vc = bf_lo(rv1[u][j]), vd = bf_hi(rv1[u][j]);
                o1[2 * j] = fmaf(p1, va, o1[2 * j]);
                o1[2 * j + 1] = fmaf(p1, vb2, o1[2 * j + 1]);
                o1[8 + 2 * j] = fmaf(p1, vc, o1[8 + 2 * j]);
                o1[8 + 2 * j + 1] = fmaf(p1, vd, o1[8 + 2 * j + 1]);
                o2[2 * j] = fmaf(p2, va, o2[2 * j]);
                o2[2 * j + 1] = fmaf(p2, vb2, o2[2 * j + 1]);
                o2[8 + 2 * j] = fmaf(p2, vc, o2[8 + 2 * j]);
                o2[8 + 2 * j + 1] = fmaf(p2, vd, o2[8 + 2 * j + 1]);
            }
        }
    }

    // ---- merge the 8 lane groups of the wave (lanes with equal g hold equal channels)
    const int xg[3] = {(lane ^ 8) << 2, (lane ^ 16) << 2, (lane ^ 32) << 2};
    float M1 = m1, M2 = m2;
#pragma unroll
    for (int s = 0; s < 3; ++s) { M1 = fmaxf(M1, lane_xor(M1, xg[s])); M2 = fmaxf(M2, lane_xor(M2, xg[s])); }
    {
        const float f1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - M1);
        const float f2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - M2);
        l1 *= f1;
        l2 *= f2;
#pragma unroll
        for (int c = 0; c < 16; ++c) { o1[c] *= f1; o2[c] *= f2; }
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        l1 += lane_xor(l1, xg[s]);
        l2 += lane_xor(l2, xg[s]);
#pragma unroll
        for (int c = 0; c < 16; ++c) { o1[c] += lane_xor(o1[c], xg[s]); o2[c] += lane_xor(o2[c], xg[s]); }
    }

    // ---- merge the 4 waves through LDS, in wave order
    __shared__ float sm[4][4];
    __shared__ float so[4][2][kDV];
    if (kg == 0) {
#pragma unroll
        for (int c = 0; c < 16; ++c) { so[wave][0][16 * g + c] = o1[c]; so[wave][1][16 * g + c] = o2[c]; }
        if (g == 0) { sm[wave][0] = M1; sm[wave][1] = l1; sm[wave][2] = M2; sm[wave][3] = l2; }
    }
    __syncthreads();
    float* part = a.ws + (((int64_t)b * a.heads + h) * a.n_splits + split) * kPartial;
    if (tid < kDV) {
        float mm1 = sm[0][0], mm2 = sm[0][2];
        for (int w = 1; w < 4; ++w) { mm1 = fmaxf(mm1, sm[w][0]); mm2 = fmaxf(mm2, sm[w][2]); }
        float L1 = 0.f, L2 = 0.f, O1 = 0.f, O2 = 0.f;
        for (int w = 0; w < 4; ++w) {
            const float f1 = (sm[w][0] == -INFINITY) ? 0.f : fast_exp2(sm[w][0] - mm1);
            const float f2 = (sm[w][2] == -INFINITY) ? 0.f : fast_exp2(sm[w][2] - mm2);
            L1 += f1 * sm[w][1];
            L2 += f2 * sm[w][3];
            O1 += f1 * so[w][0][tid];
            O2 += f2 * so[w][1][tid];
        }
        part[4 + tid] = O1;
        part[4 + kDV + tid] = O2;
        if (tid == 0) { part[0] = mm1; part[1] = L1; part[2] = mm2; part[3] = L2; }
    }
}

__global__ __launch_bounds__(kDV) void decode_reduce_kernel(DecodeArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const float* base = a.ws + ((int64_t)b * a.heads + h) * a.n_splits * kPartial;
    float M1 = -INFINITY, M2 = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < a.n_splits; ++s) {
        M1 = fmaxf(M1, base[s * kPartial + 0]);
        M2 = fmaxf(M2, base[s * kPartial + 2]);
    }
    float L1 = 0.f, L2 = 0.f, O1 = 0.f, O2 = 0.f;
#pragma unroll 8
    for (int s = 0; s < a.n_splits; ++s) {
        const float* p = base + s * kPartial;
        const float f1 = (p[0] == -INFINITY) ? 0.f : fast_exp2(p[0] - M1);
        const float f2 = (p[2] == -INFINITY) ? 0.f : fast_exp2(p[2] - M2);
        L1 += f1 * p[1];
        L2 += f2 * p[3];
        O1 += f1 * p[4 + c];
        O2 += f2 * p[4 + kDV + c];
    }
    float o;
    {
#pragma clang fp contract(off)
        o = O1 / L1 - a.lam[h] * (O2 / L2);
    }
    if (a.epi) {
        __shared__ float red[2];
        float ss = wave_sum(o * o);
        if ((c & 63) == 0) red[c >> 6] = ss;
        __syncthreads();
        ss = red[0] + red[1];
        const float w = a.norm_w ? a.norm_w[c] : 1.f;
        o = o * (1.f / sqrtf(ss * (1.f / kDV) + a.eps)) * w * (1.f - a.lambda_init);
    }
    bf16* op = (bf16*)a.out + b * a.os[0] + (int64_t)h * a.os[2];
    op[c] = (bf16)o;
}

}  // namespace

int decode_num_splits(int batch, int heads, int cache_len) {
    const int bh = batch * heads;
    int splits = (8192 + bh - 1) / bh;
    const int max_splits = (cache_len + 255) / 256;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    int split_len = (cache_len + splits - 1) / splits;
    split_len = (split_len + 127) / 128 * 128;
    return (cache_len + split_len - 1) / split_len;
}

static int decode_split_len(int cache_len, int n_splits) {
    int split_len = (cache_len + n_splits - 1) / n_splits;
    return (split_len + 127) / 128 * 128;
}

size_t decode_workspace_bytes(int batch, int heads, int cache_len, int dv) {
    (void)dv;
    const int s = decode_num_splits(batch, heads, cache_len);
    return (size_t)batch * heads * s * kPartial * sizeof(float);
}

// ---- the workspace of the allocation-free entry point
// The split partials of diffattn_decode_noalloc live in this file-scope array instead of a
// caller's workspace: one copy per GPU the library runs on (the code object's device globals are
// created when it is loaded on that GPU and live until the process ends), kNoallocScratchBytes in
// all. Host code never uses the array's name as an address (on the host it is a stand-in
// symbol): its device address is looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

hipError_t decode_noalloc_scratch(int device, float** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* ptrs[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[device]) {
        // the caller has made `device` current: the lookup returns that device's copy
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[device] = (float*)p;
    }
    *out = ptrs[device];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a0, hipStream_t stream) {
    DecodeArgs a = a0;
    a.n_splits = decode_num_splits(a.batch, a.heads, a.cache_len);
    a.split_len = decode_split_len(a.cache_len, a.n_splits);
    hipLaunchKernelGGL(decode_split_kernel, dim3(a.n_splits, a.heads, a.batch), dim3(kSplitThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(a.heads, a.batch), dim3(kDV), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
