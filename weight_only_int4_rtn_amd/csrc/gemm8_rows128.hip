// Instantiations of the eight-wave GEMM (gemm8.h) with 128-row tiles.
#include "gemm8.h"

namespace w4a16 {

hipError_t launch_gemm8_128x256(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                                hipStream_t stream) {
    return launch_gemm8<128, 256>(a, bits, bf, staged, sk, grid, stream);
}

hipError_t launch_gemm8_128x128(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                                hipStream_t stream) {
    return launch_gemm8<128, 128>(a, bits, bf, staged, sk, grid, stream);
}

}  // namespace w4a16
