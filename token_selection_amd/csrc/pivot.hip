// Per-layer summary of the pivot statistics (StructKV section 2: entropy,
// sparsity and variance of the attention, watched layer by layer during the
// first pass to find the layer where the pattern changes phase).
//
// Rows are the window rows [L][rows] with rows = B*Hq*w and the window index
// r % w; row r sees n = N - w + 1 + (r % w) keys. One work-group per layer
// sums in double:
//   entropy            the row entropy as given,
//   sparsity           n_below / n,
//   variance           sum_p2 / n - 1 / n^2  (the variance of the row's weights),
// and writes their means over the layer's rows.

#include <stdint.h>

#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
layer_summary_kernel(int rows, int w, int64_t N, const float* entropy, const float* sum_p2, const int32_t* n_below,
                     float* summary) {
    __shared__ double red[3][kThreads];
    const int l = blockIdx.x;
    double se = 0.0, ss = 0.0, sv = 0.0;
    for (int r = threadIdx.x; r < rows; r += kThreads) {
        const int64_t o = (int64_t)l * rows + r;
        const double n = (double)(N - w + 1 + r % w);
        se += (double)entropy[o];
        ss += (double)n_below[o] / n;
        sv += (double)sum_p2[o] / n - 1.0 / (n * n);
    }
    red[0][threadIdx.x] = se;
    red[1][threadIdx.x] = ss;
    red[2][threadIdx.x] = sv;
    __syncthreads();
    for (int half = kThreads / 2; half > 0; half >>= 1) {
        if ((int)threadIdx.x < half)
            for (int m = 0; m < 3; ++m) red[m][threadIdx.x] += red[m][threadIdx.x + half];
        __syncthreads();
    }
    if (threadIdx.x < 3) summary[(int64_t)l * 3 + threadIdx.x] = (float)(red[threadIdx.x][0] / rows);
}

}  // namespace

hipError_t launch_layer_summary(int32_t L, int32_t rows, int32_t w, int64_t N, const float* entropy,
                                const float* sum_p2, const int32_t* n_below, float* summary, hipStream_t st) {
    if (L < 1 || rows < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(layer_summary_kernel, dim3((unsigned)L), dim3(kThreads), 0, st, rows, w, N, entropy, sum_p2,
                       n_below, summary);
    return hipGetLastError();
}

}  // namespace kvsel
