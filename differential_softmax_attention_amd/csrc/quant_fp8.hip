// Dynamic absmax quantisation of attention score operands to fp8 (OCP e4m3: 4 exponent bits,
// bias 7, 3 mantissa bits, largest finite 448), for the fp8 forward's Q K^T.
//
// The pages report the DIFF advantage for attention logits quantised by dynamic absmax
// post-training quantisation ("softmax can't say zero, so it subtracts", section "Outliers, and
// the low-bit claim"), at an unstated granularity; here every (batch, head) slice of a Q or K
// tensor gets its own scale:  amax = max |x|,  s = amax / 448 (1 when amax = 0),
// code = e4m3(x / s) rounded to nearest even, x ~ code * s.
// Three kernels: zero the amax buffer, per-block maxima merged with an atomic max on the fp32 bit
// pattern (exact, so the result does not depend on the order), then the conversion, which also
// writes s.
#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

constexpr int kTokPerBlock = 64;

__global__ __launch_bounds__(256) void fp8_zero_kernel(float* amax, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) amax[i] = 0.f;
}

// grid (token blocks, heads, batch): max |x| over 64 tokens x dim, merged into amax[b, h]
__global__ __launch_bounds__(256) void fp8_amax_kernel(Fp8QuantArgs a) {
    const int t0 = blockIdx.x * kTokPerBlock, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const bf16* xb = (const bf16*)a.x + b * a.xs[0] + (int64_t)h * a.xs[2];
    float m = 0.f;
    const int n = min(kTokPerBlock, a.tokens - t0) * a.dim;
    for (int e = tid; e < n; e += 256) {
        const int t = t0 + e / a.dim, c = e % a.dim;
        m = fmaxf(m, fabsf((float)xb[(int64_t)t * a.xs[1] + c]));
    }
    m = wave_max(m);
    __shared__ float red[4];
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        atomicMax((unsigned int*)&a.amax[(int64_t)b * a.heads + h], __float_as_uint(m));
    }
}

// grid (token blocks, heads, batch): codes of 64 tokens, two values per lane step
__global__ __launch_bounds__(256) void fp8_convert_kernel(Fp8QuantArgs a) {
    const int t0 = blockIdx.x * kTokPerBlock, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const float am = a.amax[(int64_t)b * a.heads + h];
    const float s = am > 0.f ? am / 448.f : 1.f;
    if (blockIdx.x == 0 && tid == 0) a.scales[(int64_t)b * a.heads + h] = s;
    const bf16* xb = (const bf16*)a.x + b * a.xs[0] + (int64_t)h * a.xs[2];
    unsigned char* ob = (unsigned char*)a.out + b * a.os[0] + (int64_t)h * a.os[2];
    const int half = a.dim / 2;
    const int n = min(kTokPerBlock, a.tokens - t0) * half;
    for (int e = tid; e < n; e += 256) {
        const int t = t0 + e / half, c = 2 * (e % half);
        const bf16* xp = xb + (int64_t)t * a.xs[1] + c;
        const float v0 = (float)xp[0] / s, v1 = (float)xp[1] / s;
        // two codes in the low 16 bits, round to nearest even
        const unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        *(unsigned short*)(ob + (int64_t)t * a.os[1] + c) = (unsigned short)(w & 0xffffu);
    }
}

}  // namespace

hipError_t launch_quantize_fp8(const Fp8QuantArgs& a, hipStream_t stream) {
    const int nbh = a.batch * a.heads;
    hipLaunchKernelGGL(fp8_zero_kernel, dim3((nbh + 255) / 256), dim3(256), 0, stream, a.amax, nbh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((a.tokens + kTokPerBlock - 1) / kTokPerBlock, a.heads, a.batch);
    hipLaunchKernelGGL(fp8_amax_kernel, grid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fp8_convert_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
