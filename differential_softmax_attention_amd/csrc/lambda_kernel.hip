// lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init, one value per row of the four [n, dim]
// vector sets ("Differential Transformer: Noise-Canceling Attention by Subtraction", section
// "Making lambda learnable and stable"). One wave per row; fp32 dot products and expf.
#include "common.hpp"
#include "kernels.hpp"

namespace diffattn {

namespace {

__global__ __launch_bounds__(64) void lambda_kernel(const float* lq1, const float* lk1, const float* lq2,
                                                    const float* lk2, int dim, float lambda_init, float* out) {
    const int r = blockIdx.x, lane = threadIdx.x;
    const int64_t base = (int64_t)r * dim;
    float d1 = 0.f, d2 = 0.f;
    for (int c = lane; c < dim; c += 64) {
        d1 = fmaf(lq1[base + c], lk1[base + c], d1);
        d2 = fmaf(lq2[base + c], lk2[base + c], d2);
    }
    d1 = wave_sum(d1);
    d2 = wave_sum(d2);
    if (lane == 0) out[r] = expf(d1) - expf(d2) + lambda_init;
}

}  // namespace

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int n, int dim,
                         float lambda_init, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(lambda_kernel, dim3(n), dim3(64), 0, stream, lq1, lk1, lq2, lk2, dim, lambda_init, out);
    return hipGetLastError();
}

}  // namespace diffattn
