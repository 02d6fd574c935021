// Activation pre-pass for the large-M path: the activated input
// (SwiGLU from [up | gate] rows, or tanh-GELU; common.h) materialised once as
// 16-bit values [m][k] for the GEMM, whose x tiles travel straight from
// memory to LDS with no register stage to fuse into.  Same arithmetic as the
// fused staging of the small-M kernels, so every path feeds the same 16-bit
// inputs to its contraction ("Piper Kernels", section "ConvRot INT8": larger
// rows materialise the activation and keep the same semantics).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

template <int ACT, int AF>
__global__ __launch_bounds__(256) void activate_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t m,
                                                       int64_t k, uint16_t* __restrict__ out) {
    const int64_t per_row = k / 8;
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= m * per_row) return;
    const int64_t row = idx / per_row, c = (idx - row * per_row) * 8;
    const uint16_t* src = x + row * ldx + c;
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    const uint4 g = AF == kActFnSwiglu ? *reinterpret_cast<const uint4*>(src + k) : v;
    *reinterpret_cast<uint4*>(out + row * k + c) = activate8<ACT, AF>(v, g);
}

hipError_t launch_activate(const void* x, int act, int act_fn, int64_t m, int64_t k, int64_t ldx, void* out,
                           hipStream_t stream) {
    const unsigned blocks = unsigned(ceil_div(m * (k / 8), 256));
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    uint16_t* op = static_cast<uint16_t*>(out);
    const dim3 grid(blocks), block(256);
    if (act == kActBf16) {
        if (act_fn == kActFnSwiglu) activate_kernel<kActBf16, kActFnSwiglu><<<grid, block, 0, stream>>>(xp, ldx, m, k, op);
        else activate_kernel<kActBf16, kActFnGeluTanh><<<grid, block, 0, stream>>>(xp, ldx, m, k, op);
    } else {
        if (act_fn == kActFnSwiglu) activate_kernel<kActF16, kActFnSwiglu><<<grid, block, 0, stream>>>(xp, ldx, m, k, op);
        else activate_kernel<kActF16, kActFnGeluTanh><<<grid, block, 0, stream>>>(xp, ldx, m, k, op);
    }
    return hipGetLastError();
}

}  // namespace w4a16
