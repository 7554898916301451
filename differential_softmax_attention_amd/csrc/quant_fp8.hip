// Dynamic absmax quantisation of attention score operands to fp8 (OCP e4m3: 4 exponent bits,
// bias 7, 3 mantissa bits, largest finite 448), for the fp8 forward's Q K^T.
//
// The pages report the DIFF advantage for attention logits quantised by dynamic absmax
// post-training quantisation ("softmax can't say zero, so it subtracts", section "Outliers, and
// the low-bit claim"), at an unstated granularity; here every (batch, head) slice of a Q or K
// tensor gets its own scale:  amax = max |x|,  s = amax / 448 and r = 448 / amax (both 1 when
// amax = 0), code = e4m3(x * r) rounded to nearest even (one fp32 product per element), x ~ code * s.
// With at least 256 slices of up to 4096 x 128 elements, one kernel, a block per slice (amax, then
// the codes). Otherwise three: zero the amax buffer, per-block maxima merged with an atomic max on the
// fp32 bit pattern (exact, so the result does not depend on the order), then the conversion,
// which also writes s. The four operands of one forward (Q1, Q2, K1, K2) go through one launch
// when every slice fits in the registers of a 1024-thread block (16 x 16 bytes per thread): read
// once, amax, codes.
#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

constexpr int kTokPerBlock = 64;        // conversion kernel
constexpr int kAmaxTokPerBlock = 256;   // maximum kernel

__global__ __launch_bounds__(256) void fp8_zero_kernel(float* amax, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) amax[i] = 0.f;
}

// grid (token blocks, heads, batch): max |x| over 256 tokens x dim, merged into amax[b, h].
// VEC: 8 elements (16 bytes) per thread step.
template <bool VEC>
__global__ __launch_bounds__(256) void fp8_amax_kernel(Fp8QuantArgs a) {
    const int t0 = blockIdx.x * kAmaxTokPerBlock, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const bf16* xb = (const bf16*)a.x + b * a.xs[0] + (int64_t)h * a.xs[2];
    float m = 0.f;
    if (VEC) {
        // eight independent 16-byte loads in flight per thread (past the end: the last chunk again)
        const int cpr = a.dim / 8;
        const int n = min(kAmaxTokPerBlock, a.tokens - t0) * cpr;
        constexpr int U = 8;
        for (int e0 = tid; e0 < n; e0 += 256 * U) {
            bf16x8 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = min(e0 + u * 256, n - 1);
                v[u] = *(const bf16x8*)(xb + (int64_t)(t0 + e / cpr) * a.xs[1] + 8 * (e % cpr));
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)v[u][j]));
        }
    } else {
        const int n = min(kAmaxTokPerBlock, a.tokens - t0) * a.dim;
        for (int e = tid; e < n; e += 256) {
            const int t = t0 + e / a.dim, c = e % a.dim;
            m = fmaxf(m, fabsf((float)xb[(int64_t)t * a.xs[1] + c]));
        }
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

// grid (token blocks, heads, batch): codes of 64 tokens, two values per lane step (VEC: eight)
template <bool VEC>
__global__ __launch_bounds__(256) void fp8_convert_kernel(Fp8QuantArgs a) {
    const int t0 = blockIdx.x * kTokPerBlock, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const float am = a.amax[(int64_t)b * a.heads + h];
    const float s = am > 0.f ? am / 448.f : 1.f;
    const float r = am > 0.f ? 448.f / am : 1.f;
    if (blockIdx.x == 0 && tid == 0) a.scales[(int64_t)b * a.heads + h] = s;
    const bf16* xb = (const bf16*)a.x + b * a.xs[0] + (int64_t)h * a.xs[2];
    unsigned char* ob = (unsigned char*)a.out + b * a.os[0] + (int64_t)h * a.os[2];
    if (VEC) {
        const int cpr = a.dim / 8;
        const int n = min(kTokPerBlock, a.tokens - t0) * cpr;
        for (int e = tid; e < n; e += 256) {
            const int t = t0 + e / cpr, c = 8 * (e % cpr);
            const bf16x8 v = *(const bf16x8*)(xb + (int64_t)t * a.xs[1] + c);
            unsigned w[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // codes 4j .. 4j+3: low word then high word of one 32-bit value
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[4 * j] * r, (float)v[4 * j + 1] * r, 0, false);
                w[j] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32((float)v[4 * j + 2] * r, (float)v[4 * j + 3] * r, lo, true);
            }
            *(uint2*)(ob + (int64_t)t * a.os[1] + c) = make_uint2(w[0], w[1]);
        }
        return;
    }
    const int half = a.dim / 2;
    const int n = min(kTokPerBlock, a.tokens - t0) * half;
    for (int e = tid; e < n; e += 256) {
        const int t = t0 + e / half, c = 2 * (e % half);
        const bf16* xp = xb + (int64_t)t * a.xs[1] + c;
        const float v0 = (float)xp[0] * r, v1 = (float)xp[1] * r;
        // two codes in the low 16 bits, round to nearest even
        const unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        *(unsigned short*)(ob + (int64_t)t * a.os[1] + c) = (unsigned short)(w & 0xffffu);
    }
}

// One block per (head, batch) slice (short slices): the slice's amax, then its codes, in one
// launch and without atomics; the second pass reads the slice again, mostly from L2.
__global__ __launch_bounds__(1024) void fp8_slice_kernel(Fp8QuantArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const bf16* xb = (const bf16*)a.x + b * a.xs[0] + (int64_t)h * a.xs[2];
    unsigned char* ob = (unsigned char*)a.out + b * a.os[0] + (int64_t)h * a.os[2];
    const int cpr = a.dim / 8;
    const int n = a.tokens * cpr;
    float m = 0.f;
    // eight independent 16-byte loads in flight per thread
    constexpr int U = 8;
    for (int e0 = tid; e0 < n; e0 += 1024 * U) {
        bf16x8 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = min(e0 + u * 1024, n - 1);   // past the end: reread the last chunk
            v[u] = *(const bf16x8*)(xb + (int64_t)(e / cpr) * a.xs[1] + 8 * (e % cpr));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)v[u][j]));
    }
    m = wave_max(m);
    __shared__ float red[16];
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    float am = red[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) am = fmaxf(am, red[w]);
    const float s = am > 0.f ? am / 448.f : 1.f;
    const float r = am > 0.f ? 448.f / am : 1.f;
    if (tid == 0) {
        a.amax[(int64_t)b * a.heads + h] = am;
        a.scales[(int64_t)b * a.heads + h] = s;
    }
    for (int e0 = tid; e0 < n; e0 += 1024 * U) {
        bf16x8 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = min(e0 + u * 1024, n - 1);
            v[u] = *(const bf16x8*)(xb + (int64_t)(e / cpr) * a.xs[1] + 8 * (e % cpr));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * 1024;
            if (e >= n) break;
            const int t = e / cpr, c = 8 * (e % cpr);
            unsigned w[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[u][4 * j] * r, (float)v[u][4 * j + 1] * r, 0, false);
                w[j] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32((float)v[u][4 * j + 2] * r, (float)v[u][4 * j + 3] * r, lo,
                                                                 true);
            }
            *(uint2*)(ob + (int64_t)t * a.os[1] + c) = make_uint2(w[0], w[1]);
        }
    }
}

// Several operands in one launch, one block per (head, batch, operand) slice of up to
// 1024 x kRegChunks 16-byte chunks, held in registers between its two steps: the slice is read
// once from memory, its amax taken (wave and block reductions, no atomics), then its codes written
// from the registers.
constexpr int kRegChunks = 16;
__global__ __launch_bounds__(1024) void fp8_slices_reg_kernel(Fp8QuantManyArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, op = blockIdx.z;
    const int tid = threadIdx.x;
    const bf16* xb = (const bf16*)a.x[op] + b * a.xs[op][0] + (int64_t)h * a.xs[op][2];
    unsigned char* ob = (unsigned char*)a.out[op] + b * a.os[op][0] + (int64_t)h * a.os[op][2];
    const int64_t xt = a.xs[op][1], ot = a.os[op][1];
    const int cpr = a.dim / 8;
    const int n = a.tokens[op] * cpr;
    bf16x8 v[kRegChunks];
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) {
        const int e = min(tid + u * 1024, n - 1);   // past the end: the last chunk again
        v[u] = *(const bf16x8*)(xb + (int64_t)(e / cpr) * xt + 8 * (e % cpr));
    }
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)v[u][j]));
    m = wave_max(m);
    __shared__ float red[16];
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    float am = red[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) am = fmaxf(am, red[w]);
    const float s = am > 0.f ? am / 448.f : 1.f;
    const float r = am > 0.f ? 448.f / am : 1.f;
    if (tid == 0) {
        a.amax[op][(int64_t)b * a.heads + h] = am;
        a.scales[op][(int64_t)b * a.heads + h] = s;
    }
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) {
        const int e = tid + u * 1024;
        if (e < n) {
            const int t = e / cpr, c = 8 * (e % cpr);
            unsigned w[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32((float)v[u][4 * j] * r, (float)v[u][4 * j + 1] * r, 0, false);
                w[j] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32((float)v[u][4 * j + 2] * r, (float)v[u][4 * j + 3] * r,
                                                                 lo, true);
            }
            *(uint2*)(ob + (int64_t)t * ot + c) = make_uint2(w[0], w[1]);
        }
    }
}

bool fp8_vec_ok(const void* x, const int64_t* xs, const void* out, const int64_t* os, int dim) {
    return dim % 8 == 0 && ((uintptr_t)x) % 16 == 0 && xs[0] % 8 == 0 && xs[1] % 8 == 0 && xs[2] % 8 == 0 &&
           ((uintptr_t)out) % 8 == 0 && os[0] % 8 == 0 && os[1] % 8 == 0 && os[2] % 8 == 0;
}

}  // namespace

hipError_t launch_quantize_fp8_many(const Fp8QuantManyArgs& a, hipStream_t stream) {
    bool one = true;
    for (int i = 0; i < a.n; ++i)
        one = one && fp8_vec_ok(a.x[i], a.xs[i], a.out[i], a.os[i], a.dim) &&
              (int64_t)a.tokens[i] * (a.dim / 8) <= (int64_t)1024 * kRegChunks;
    if (one) {
        hipLaunchKernelGGL(fp8_slices_reg_kernel, dim3(a.heads, a.batch, a.n), dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    // longer slices: each operand on its own
    for (int i = 0; i < a.n; ++i) {
        Fp8QuantArgs s{};
        s.x = a.x[i];
        s.out = a.out[i];
        for (int k = 0; k < 3; ++k) { s.xs[k] = a.xs[i][k]; s.os[k] = a.os[i][k]; }
        s.scales = a.scales[i];
        s.amax = a.amax[i];
        s.batch = a.batch; s.tokens = a.tokens[i]; s.heads = a.heads; s.dim = a.dim;
        if (hipError_t e = launch_quantize_fp8(s, stream)) return e;
    }
    return hipSuccess;
}

hipError_t launch_quantize_fp8(const Fp8QuantArgs& a, hipStream_t stream) {
    const bool vec = fp8_vec_ok(a.x, a.xs, a.out, a.os, a.dim);
    if (vec && (int64_t)a.tokens * a.dim <= (int64_t)4096 * 128 && a.batch * a.heads >= 256) {
        hipLaunchKernelGGL(fp8_slice_kernel, dim3(a.heads, a.batch), dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    const int nbh = a.batch * a.heads;
    hipLaunchKernelGGL(fp8_zero_kernel, dim3((nbh + 255) / 256), dim3(256), 0, stream, a.amax, nbh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // longer slices: per-block maxima merged by an atomic max, then the conversion; 16-byte reads
    // and 8-byte code stores when every row of the slice allows them
    const dim3 grid((a.tokens + kTokPerBlock - 1) / kTokPerBlock, a.heads, a.batch);
    const dim3 agrid((a.tokens + kAmaxTokPerBlock - 1) / kAmaxTokPerBlock, a.heads, a.batch);
    if (vec) hipLaunchKernelGGL(fp8_amax_kernel<true>, agrid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(fp8_amax_kernel<false>, agrid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (vec) hipLaunchKernelGGL(fp8_convert_kernel<true>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(fp8_convert_kernel<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace diffattn
