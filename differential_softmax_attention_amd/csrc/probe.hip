// Measurement helpers: the attainable dense bf16 MFMA rate of the device, against which the
// kernels' algorithmic throughput can be read beside the published peak.
#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

// Each wave keeps 8 independent accumulator chains of v_mfma_f32_32x32x16_bf16 busy; operands
// come from registers only.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (bf16)(0.001f * (lane + j));
        b[j] = (bf16)(0.002f * (lane - j));
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
    return hipGetLastError();
}

}  // namespace diffattn
