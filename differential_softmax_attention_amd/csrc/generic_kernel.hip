// Generic differential-attention kernel: any dtype (fp32 or bf16 storage, fp32 arithmetic), any
// d <= 256 and dv <= 512, V1 prefill, V1 decode and V2 pairs through one head mapping.
//
// It computes, per output row, O = (softmax(s q1 K1^T) - lambda softmax(s q2 K2^T)) V over the
// visible keys, then the optional RMSNorm * w * (1 - lambda_init) epilogue
// ("Differential Transformer: Noise-Canceling Attention by Subtraction", sections "The mechanism"
// and "Making lambda learnable and stable").
//
// One 64-lane wave owns one output row. Keys are taken 64 at a time: lane j scores key j of the
// chunk for both maps, the chunk's maxima and sums are reduced across the wave and folded into
// the running (max, sum) of each map, and each lane then accumulates its own output channels
// (c = lane, lane + 64, ...) over the chunk. exp is the accurate expf, so fp32 inputs meet a
// 1e-5 absolute tolerance.
#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

constexpr int kMaxD = 256;
constexpr int kMaxDvPerLane = 8;  // dv <= 512

template <typename T>
__global__ __launch_bounds__(64) void generic_diffattn_kernel(GenericArgs a) {
    const int i = blockIdx.x;   // query row
    const int h = blockIdx.y;   // output head
    const int b = blockIdx.z;
    const int lane = threadIdx.x;

    __shared__ float sq1[kMaxD];
    __shared__ float sq2[kMaxD];
    __shared__ float sp1[64];
    __shared__ float sp2[64];

    const T* q1 = (const T*)a.q1 + b * a.q1s[0] + (int64_t)i * a.q1s[1] + (int64_t)(h * a.q_hmul + a.q1_hoff) * a.q1s[2];
    const T* q2 = (const T*)a.q2 + b * a.q2s[0] + (int64_t)i * a.q2s[1] + (int64_t)(h * a.q_hmul + a.q2_hoff) * a.q2s[2];
    for (int c = lane; c < a.d; c += 64) {
        sq1[c] = to_f32(q1[c]);
        sq2[c] = to_f32(q2[c]);
    }
    __syncthreads();

    int nk = a.seq_k;
    if (a.key_lens) nk = min(max(a.key_lens[b], 1), a.seq_k);
    int nvis = nk;
    if (a.causal) nvis = min(nk, i + (nk - a.seq_q) + 1);

    const int kvh = (h * a.q_hmul) / a.kv_hdiv;
    const T* k1 = (const T*)a.k1 + b * a.k1s[0] + (int64_t)kvh * a.k1s[2];
    const T* k2 = (const T*)a.k2 + b * a.k2s[0] + (int64_t)kvh * a.k2s[2];
    const T* v = (const T*)a.v + b * a.vs[0] + (int64_t)kvh * a.vs[2];

    float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f;
    float o1[kMaxDvPerLane], o2[kMaxDvPerLane];
#pragma unroll
    for (int t = 0; t < kMaxDvPerLane; ++t) { o1[t] = 0.f; o2[t] = 0.f; }

    for (int j0 = 0; j0 < nvis; j0 += 64) {
        const int j = j0 + lane;
        float s1 = -INFINITY, s2 = -INFINITY;
        if (j < nvis) {
            const T* k1r = k1 + (int64_t)j * a.k1s[1];
            const T* k2r = k2 + (int64_t)j * a.k2s[1];
            float acc1 = 0.f, acc2 = 0.f;
            for (int c = 0; c < a.d; ++c) {
                acc1 = fmaf(sq1[c], to_f32(k1r[c]), acc1);
                acc2 = fmaf(sq2[c], to_f32(k2r[c]), acc2);
            }
            s1 = acc1 * a.scale;
            s2 = acc2 * a.scale;
        }
        // chunk maxima; the chunk's first key is always visible, so they are finite
        const float mn1 = fmaxf(m1, wave_max(s1));
        const float mn2 = fmaxf(m2, wave_max(s2));
        const float p1 = (j < nvis) ? expf(s1 - mn1) : 0.f;
        const float p2 = (j < nvis) ? expf(s2 - mn2) : 0.f;
        const float al1 = expf(m1 - mn1);   // 0 on the first chunk (m = -inf)
        const float al2 = expf(m2 - mn2);
        l1 = l1 * al1 + wave_sum(p1);
        l2 = l2 * al2 + wave_sum(p2);
        m1 = mn1;
        m2 = mn2;
        sp1[lane] = p1;
        sp2[lane] = p2;
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kMaxDvPerLane; ++t) { o1[t] *= al1; o2[t] *= al2; }
        const int cnt = min(64, nvis - j0);
        for (int jj = 0; jj < cnt; ++jj) {
            const T* vr = v + (int64_t)(j0 + jj) * a.vs[1];
            const float w1 = sp1[jj], w2 = sp2[jj];
#pragma unroll
            for (int t = 0; t < kMaxDvPerLane; ++t) {
                const int c = lane + 64 * t;
                if (c < a.dv) {
                    const float x = to_f32(vr[c]);
                    o1[t] = fmaf(w1, x, o1[t]);
                    o2[t] = fmaf(w2, x, o2[t]);
                }
            }
        }
        __syncthreads();
    }

    const float lam_raw = a.lam[b * a.lams[0] + (int64_t)i * a.lams[1] + (int64_t)h * a.lams[2]];
    const float lam = a.lam_sigmoid ? sigmoid_f32(lam_raw) : lam_raw;
    const float r1 = 1.f / l1, r2 = 1.f / l2;
    float o[kMaxDvPerLane];
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < kMaxDvPerLane; ++t) {
#pragma clang fp contract(off)
        o[t] = o1[t] * r1 - lam * (o2[t] * r2);
        if (lane + 64 * t < a.dv) ss = fmaf(o[t], o[t], ss);
    }
    if (a.epi) {
        ss = wave_sum(ss);
        const float inv = 1.f / sqrtf(ss / (float)a.dv + a.eps);
        const float post = 1.f - a.lambda_init;
#pragma unroll
        for (int t = 0; t < kMaxDvPerLane; ++t) {
            const int c = lane + 64 * t;
            const float w = (a.norm_w && c < a.dv) ? a.norm_w[c] : 1.f;
            o[t] = o[t] * inv * w * post;
        }
    }
    T* out = (T*)a.out + b * a.os[0] + (int64_t)i * a.os[1] + (int64_t)h * a.os[2];
#pragma unroll
    for (int t = 0; t < kMaxDvPerLane; ++t) {
        const int c = lane + 64 * t;
        if (c < a.dv) out[c] = from_f32<T>(o[t]);
    }
}

}  // namespace

hipError_t launch_generic(const GenericArgs& a, int batch, int heads, bool bf16_io, hipStream_t stream) {
    dim3 grid(a.seq_q, heads, batch);
    if (bf16_io)
        hipLaunchKernelGGL(generic_diffattn_kernel<bf16>, grid, dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL(generic_diffattn_kernel<float>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
