// Split-K reduce: y[m][n] = round(sum_s partials[s][m][n] + bias[n]).
//
// The K-split kernels store FP32 partial sums of each split; this kernel adds
// them in split order (so results are reproducible), adds the bias in FP32
// once and rounds once to the output dtype ("Piper Kernels", section "NVFP4
// construction": bias applied in FP32 before the final 16-bit conversion).
// A separate launch replaces inter-workgroup synchronisation, whose
// device-scope fences would write back and invalidate the L2 of every XCD.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

template <int ACT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials, int splits,
                                                            int64_t m, int64_t n, int64_t npad,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, int64_t ldy) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= m * n) return;
    const int64_t row = idx / n, col = idx - row * n;
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) v += partials[(int64_t(s) * m + row) * npad + col];
    if (bias) v += to_f32<ACT>(bias[col]);
    y[row * ldy + col] = from_f32<ACT>(v);
}

hipError_t launch_splitk_reduce(const float* partials, int splits, int64_t m, int64_t n, int64_t npad,
                                const uint16_t* bias, uint16_t* y, int64_t ldy, int act,
                                hipStream_t stream) {
    const unsigned blocks = unsigned(ceil_div(m * n, 256));
    if (act == kActBf16)
        splitk_reduce_kernel<kActBf16><<<dim3(blocks), dim3(256), 0, stream>>>(partials, splits, m, n, npad,
                                                                               bias, y, ldy);
    else
        splitk_reduce_kernel<kActF16><<<dim3(blocks), dim3(256), 0, stream>>>(partials, splits, m, n, npad,
                                                                              bias, y, ldy);
    return hipGetLastError();
}

}  // namespace w4a16
