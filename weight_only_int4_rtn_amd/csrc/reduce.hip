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

// One thread per 4 consecutive outputs of a row: 16-byte partial loads (npad
// is a multiple of 4 and the partials 16-byte aligned); an 8-byte store when
// the output row allows it, element stores otherwise and at a ragged end.
template <int ACT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials, int splits,
                                                            int64_t m, int64_t n, int64_t npad,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, int64_t ldy, int vec_store) {
    const int64_t quads = (n + 3) / 4;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= m * quads) return;
    const int64_t row = idx / quads, c0 = (idx - row * quads) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < splits; ++s) {
        const float4 p = *reinterpret_cast<const float4*>(partials + (int64_t(s) * m + row) * npad + c0);
        v.x += p.x;
        v.y += p.y;
        v.z += p.z;
        v.w += p.w;
    }
    float o[4] = {v.x, v.y, v.z, v.w};
    const int cnt = int(min<int64_t>(4, n - c0));
    if (bias) {
        for (int e = 0; e < cnt; ++e) o[e] += to_f32<ACT>(bias[c0 + e]);
    }
    uint16_t* yr = y + row * ldy + c0;
    if (cnt == 4 && vec_store) {
        *reinterpret_cast<uint2*>(yr) =
            make_uint2(uint32_t(from_f32<ACT>(o[0])) | (uint32_t(from_f32<ACT>(o[1])) << 16),
                       uint32_t(from_f32<ACT>(o[2])) | (uint32_t(from_f32<ACT>(o[3])) << 16));
    } else {
        for (int e = 0; e < cnt; ++e) yr[e] = from_f32<ACT>(o[e]);
    }
}

hipError_t launch_splitk_reduce(const float* partials, int splits, int64_t m, int64_t n, int64_t npad,
                                const uint16_t* bias, uint16_t* y, int64_t ldy, int act,
                                hipStream_t stream) {
    const unsigned blocks = unsigned(ceil_div(m * ceil_div(n, 4), 256));
    // 8-byte stores need every row start 8-byte aligned
    const int vec_store = reinterpret_cast<uintptr_t>(y) % 8 == 0 && ldy % 4 == 0;
    if (act == kActBf16)
        splitk_reduce_kernel<kActBf16><<<dim3(blocks), dim3(256), 0, stream>>>(partials, splits, m, n, npad,
                                                                               bias, y, ldy, vec_store);
    else
        splitk_reduce_kernel<kActF16><<<dim3(blocks), dim3(256), 0, stream>>>(partials, splits, m, n, npad,
                                                                              bias, y, ldy, vec_store);
    return hipGetLastError();
}

}  // namespace w4a16
