// Launchers and launch plans of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// Workspace = [arrival counters: kMaxSlots uint32][FP32 partial sums].
// The counter region has a fixed size so that partial sums of one call can
// never land on the counters of a later call with another shape: counters
// start zeroed (the caller zero-fills a new workspace) and every call leaves
// the counters it used at zero.  A launch uses at most kMaxSlots counters.
constexpr int64_t kMaxSlots = 16384;
constexpr size_t kCounterBytes = size_t(kMaxSlots) * 4;
inline size_t workspace_layout_bytes(size_t partial_floats) {
    return kCounterBytes + partial_floats * 4;
}
inline float* workspace_partials(void* ws) {
    return reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kCounterBytes);
}

struct GemvPlan {
    int gps, splits;
    int64_t tiles_per_launch;  // tile range of one launch (<= kMaxSlots when split)
    size_t lds, workspace;
};
GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k);

struct SkinnyPlan {
    int mb;             // 16-row m-subtiles per workgroup (1..4)
    int gps, splits;
    int64_t tile_groups, mblocks;
    size_t workspace;
};
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k);

struct GemmPlan {
    int64_t mtiles, ntiles;
    size_t workspace;
};
GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k);

hipError_t launch_quantize(const void* w, int dtype, int64_t n, int64_t k, int64_t ldw,
                           uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_pack(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                       void* packed, hipStream_t stream);
hipError_t launch_unpack(const void* packed, int64_t n, int64_t k, uint8_t* codes, float* scales,
                         hipStream_t stream);

// m <= 4 per launch (the caller splits larger m into row blocks).
hipError_t launch_gemv(const void* x, int act, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream);
hipError_t launch_skinny(const void* x, int act, int64_t m, int64_t k, int64_t ldx, const void* packed,
                         int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                         hipStream_t stream);
hipError_t launch_gemm(const void* x, int act, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream);

}  // namespace w4a16
