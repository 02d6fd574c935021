// Launchers and launch plans of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

namespace w4a16 {

// Workspace of a K-split launch: a header of kSyncBytes holding the 64-bit
// exchange slots through which small-M launches finish their split in-kernel
// (or the 32-bit tile counters of the mid-M and stream-K launches), then
// FP32 partial sums [splits][m][npad] for the split-K reduce kernel (or the
// tile slots those launches add in-kernel).  The header must be zero before
// a call and every call leaves it zero (the thread that empties a slot, or
// completes a count, clears it); the partial sums need no initialisation
// (every element that reaches an output is written first; the reduce kernel
// also reads, and drops, the padding columns past n of a 4-column group).
// Every path places its partial sums after the header.
constexpr size_t kSyncBytes = size_t(1) << 20;

struct GemvPlan {
    int waves, gps, splits, cpw;  // cpw: chunks each wave loads up front
    bool exchange;                // split finished through the header's exchange slots
    size_t lds, workspace;
};
// bits: 4 (INT4 packed weights) or 8 (INT8)
GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k, int bits = 4);

struct MgemvPlan {
    int mmax, waves, gps, splits, cpw;
    bool direct;    // x operands loaded with each chunk, else staged in LDS
    bool exchange;  // split finished through the header's exchange slots
    size_t lds, workspace;
};
MgemvPlan plan_mgemv(int64_t m, int64_t n, int64_t k, int bits = 4, int act_fn = 0);

struct SkinnyPlan {
    int mb;             // 16-row m-subtiles per workgroup (1..4)
    int waves;          // waves per workgroup, one 16-row weight tile each
    bool direct;        // x slice whole in LDS (no fused activation), else staged per group
    int gps, splits;
    int gmax;           // register capacity for chunks (4, 8, 16 groups)
    int64_t tile_groups, mblocks;
    bool in_kernel;     // a K split finished inside the launch (else by the reduce kernel)
    size_t workspace;
};
// act_fn: ActFn (common.h) fused into the input
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int bits, int act_fn);

struct GemmPlan {
    int64_t mtiles, ntiles;
    int waves;            // 8: the eight-wave kernel (bm x bn tiles); 4: the four-wave kernel (bm x 256)
    int bm, bn;           // workgroup tile: rows of x, output columns
    int mb, gps, splits;  // mb = bm / 16; gps: groups per K split
    bool sk;              // stream-K: wgs workgroups, each a run of tiles x groups units (splits 1)
    int64_t wgs;          // workgroups of the launch
    size_t workspace;
};
GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, int bits = 4);
// stream-K plans: a given tile, and the modelled fastest stream-K tile
GemmPlan plan_gemm_sk(int64_t m, int64_t n, int64_t k, int bits, int bm, int bn, int64_t runs);
GemmPlan plan_gemm_streamk(int64_t m, int64_t n, int64_t k, int bits);

// One launch of a path's main kernel, as w4a16_linear_explain reports it.
struct PlanInfo {
    int waves;           // waves (64 lanes) per workgroup
    int tile_m, tile_n;  // x rows and output columns one workgroup computes
    int splits, gps;     // K parts, 128-column groups per part
    int64_t workgroups;  // grid size
    bool reduce;         // a split-K reduce launch follows
    bool stream_k;       // stream-K: splits = the most runs sharing a tile, gps = the longest run
};
PlanInfo describe_gemv(int64_t m, int64_t n, int64_t k, int bits);    // m <= 4 (one row block)
PlanInfo describe_mgemv(int64_t m, int64_t n, int64_t k, int bits, int act_fn);   // m <= 16 (one row block)
PlanInfo describe_skinny(int64_t m, int64_t n, int64_t k, int bits, int act_fn);
PlanInfo describe_gemm(int64_t m, int64_t n, int64_t k, int bits, bool streamk);

hipError_t launch_quantize(const void* w, int dtype, int64_t n, int64_t k, int64_t ldw,
                           uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_pack(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                       void* packed, hipStream_t stream);
hipError_t launch_unpack(const void* packed, int64_t n, int64_t k, uint8_t* codes, float* scales,
                         hipStream_t stream);
// INT8: codes [n][k] one signed code per byte.
hipError_t launch_quantize8(const void* w, int dtype, int64_t n, int64_t k, int64_t ldw, int8_t* codes,
                            float* scales, hipStream_t stream);
hipError_t launch_pack8(const int8_t* codes, const float* scales, int64_t n, int64_t k, void* packed,
                        hipStream_t stream);
hipError_t launch_unpack8(const void* packed, int64_t n, int64_t k, int8_t* codes, float* scales,
                          hipStream_t stream);
// In place: packed <- requantize(beta * dequant(packed) + alpha * U), U the
// dense update [n][ldu] (rank 0) or mat1 [n][rank] @ mat2 [rank][k]; dtype
// 0 (FP32), kActBf16 or kActF16; stochastic rounding with `seed` when set.
hipError_t launch_update(void* packed, int64_t n, int64_t k, const void* upd, int64_t ldu, const void* mat1,
                         const void* mat2, int64_t rank, int dtype, float alpha, float beta, int stochastic,
                         uint64_t seed, int bits, hipStream_t stream);
// Rows [start, start + len) (dim 0) or group-aligned columns (dim 1) of a
// packed [n][k] weight (bits 4 or 8) into a new packed weight.
hipError_t launch_shard(const void* packed, int64_t n, int64_t k, int dim, int64_t start, int64_t len,
                        void* out, int bits, hipStream_t stream);

// y[m][n] = round(sum over splits of partials[s][m][npad] + bias): finishes K-split launches.
hipError_t launch_splitk_reduce(const float* partials, int splits, int64_t m, int64_t n, int64_t npad,
                                const uint16_t* bias, uint16_t* y, int64_t ldy, int act,
                                hipStream_t stream);

// act_fn (ActFn, common.h): activation fused into the x staging; SwiGLU x
// rows hold [up | gate], 2k values.
// bits: 4 or 8 (packed INT4 or INT8 weights).
// m <= 4 per launch (the caller splits larger m into row blocks).
hipError_t launch_gemv(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                       const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream);
// m <= 16 per launch (the caller splits larger m into row blocks); bits 4 or 8.
hipError_t launch_mgemv(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                        const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                        hipStream_t stream);
hipError_t launch_skinny(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                         const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                         hipStream_t stream);
// The activated input [m][k] (row stride k) of x for the GEMM path.
hipError_t launch_activate(const void* x, int act, int act_fn, int64_t m, int64_t k, int64_t ldx, void* out,
                           hipStream_t stream);
// streamk: the stream-K decomposition (on the planner's tile, or the nearest
// one it offers) instead of the planner's choice
hipError_t launch_gemm(const void* x, int act, int bits, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace, bool streamk,
                       hipStream_t stream);

// The argument checks of w4a16_linear alone (its status before any launch;
// OK means the call would launch or is a no-op).  Declared here so other
// entry points of the library can validate before their own set-up.
w4a16_status_t check_linear(const void* x, w4a16_dtype_t act_dtype, int64_t m, int64_t k, int64_t ldx,
                            const void* packed, int64_t n, const void* bias, void* y, int64_t ldy,
                            void* workspace, size_t workspace_bytes);

}  // namespace w4a16
