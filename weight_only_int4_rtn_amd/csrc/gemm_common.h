// Definitions shared by the large-M GEMM kernels (gemm.hip, gemm8.h): the
// launch arguments, the inline-asm MFMA with its accumulator in AGPRs, the
// bias load, 16-bit packing and the dequantization of packed words.
#pragma once

#include "common.h"
#include "kernels.h"

namespace w4a16 {

struct GemmArgs {
    const uint16_t* x;
    int64_t ldx, m;
    const uint8_t* packed;
    int64_t n, k;
    const uint16_t* bias;
    uint16_t* y;
    int64_t ldy;
    float* partials;  // [splits][m][ntiles * tile columns] when splits > 1; stream-K: slots of FP32 tile sums
    int splits, gps;
    int vec_store;    // y 8-byte aligned and ldy % 4 == 0: 4 outputs per store
    int vec16;        // y 16-byte aligned and ldy % 8 == 0: 8 outputs per store
    int64_t mtiles, ntiles;
    unsigned* counters;  // stream-K: a counter per tile in the workspace header (zero between calls)
    int64_t sk_units;    // stream-K: tiles x 128-column groups (0: not stream-K)
};

// D = A . B + C on v_mfma_f32_16x16x32_{bf16,f16} through the compiler
// builtin (the compiler places accumulators and pads hazards).
template <int ACT>
__device__ inline f32x4_t gm_mfma(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (ACT == kActBf16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
}

// Bias of the four output columns c0 .. c0 + 3 of each of a lane's T
// 16-column tiles (t0 .. t0 + T - 1), in FP32, zero past n or without a
// bias.  The loads use clamped indices and no branches, so all of them are
// in flight together (element-wise conditional loads were each waited for
// before the next was issued).
template <int ACT, int T>
__device__ inline void bias_tiles(const uint16_t* bias, int64_t t0, int kq, int64_t n, float (&bv)[T][4]) {
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[j][e] = 0.0f;
    if (!bias) return;
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t c = (t0 + j) * 16 + 4 * kq + e;
            const float v = to_f32<ACT>(bias[c < n ? c : n - 1]);
            bv[j][e] = c < n ? v : 0.0f;
        }
}

// Two FP32 values -> packed pair of the 16-bit type, round to nearest even
// (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <int ACT>
__device__ inline uint32_t pack2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    if constexpr (ACT == kActBf16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Byte B of a word as a float: one v_cvt_f32_ubyteB (left to itself the
// compiler re-extracts each nibble with a v_bfe_u32 first).
template <int B>
__device__ inline float byte_f32(uint32_t w) {
    float f;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(w));
    else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(w));
    else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(w));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(w));
    return f;
}

// One packed word (8 codes of columns j = 0..7, nibble i = column 2i, nibble
// i + 4 = column 2i + 1) -> 8 dequantized 16-bit values in column order:
// 3 bit operations, 8 conversions, 8 fma and 4 packs.
template <int ACT>
__device__ inline uint4 dequant_word(uint32_t w, float s, float neg8s) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // bytes: columns 0, 4, 1, 5
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // bytes: columns 2, 6, 3, 7
    const float c0 = fmaf(byte_f32<0>(lo), s, neg8s);
    const float c4 = fmaf(byte_f32<1>(lo), s, neg8s);
    const float c1 = fmaf(byte_f32<2>(lo), s, neg8s);
    const float c5 = fmaf(byte_f32<3>(lo), s, neg8s);
    const float c2 = fmaf(byte_f32<0>(hi), s, neg8s);
    const float c6 = fmaf(byte_f32<1>(hi), s, neg8s);
    const float c3 = fmaf(byte_f32<2>(hi), s, neg8s);
    const float c7 = fmaf(byte_f32<3>(hi), s, neg8s);
    return make_uint4(pack2<ACT>(c0, c1), pack2<ACT>(c2, c3), pack2<ACT>(c4, c5), pack2<ACT>(c6, c7));
}

// Two INT8 words (columns 0-3 and 4-7, byte b = column b, u = q + 128) ->
// 8 dequantized 16-bit values in column order: fma(u, s, -128 s), -128 s
// exact.
template <int ACT>
__device__ inline uint4 dequant_word8(uint32_t w0, uint32_t w1, float s, float neg128s) {
    return make_uint4(pack2<ACT>(fmaf(byte_f32<0>(w0), s, neg128s), fmaf(byte_f32<1>(w0), s, neg128s)),
                      pack2<ACT>(fmaf(byte_f32<2>(w0), s, neg128s), fmaf(byte_f32<3>(w0), s, neg128s)),
                      pack2<ACT>(fmaf(byte_f32<0>(w1), s, neg128s), fmaf(byte_f32<1>(w1), s, neg128s)),
                      pack2<ACT>(fmaf(byte_f32<2>(w1), s, neg128s), fmaf(byte_f32<3>(w1), s, neg128s)));
}

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// The eight-wave kernel's launchers, one per workgroup tile (rows x
// columns), defined in gemm8_rows256.hip and gemm8_rows128.hip.
hipError_t launch_gemm8_256x256(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                                hipStream_t stream);
hipError_t launch_gemm8_256x128(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                                hipStream_t stream);
hipError_t launch_gemm8_128x256(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                                hipStream_t stream);
hipError_t launch_gemm8_128x128(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                                hipStream_t stream);

}  // namespace w4a16
