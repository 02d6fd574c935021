// Large-M forward: placeholder plan (the LDS-staged MFMA kernel is added next).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k) {
    (void)k;
    GemmPlan p{};
    p.mtiles = ceil_div(m, 128);
    p.ntiles = ceil_div(n, 128);
    p.workspace = 0;
    return p;
}

hipError_t launch_gemm(const void*, int, int64_t, int64_t, int64_t, const void*, int64_t, const void*,
                       void*, int64_t, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace w4a16
