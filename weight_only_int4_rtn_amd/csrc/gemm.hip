// Large-M forward: the layer as a dense contraction on the matrix cores
// (v_mfma_f32_16x16x32_{bf16,f16}, FP32 accumulation).
//
// Each 16 x 16 output block is computed as D = W . x^T: the dequantized
// weights are the A operand and the x rows the B operand.  A packed chunk
// (16 output columns x 128 k, one 16-byte run per lane) is exactly an MFMA
// operand: lane L holds row L % 16 of the tile and k = 8 (L / 16) + j of each
// 32-wide k-step, one 32-bit word per k-step.  Dequantization happens once per
// word as q * s rounded once to the 16-bit input type (byte -> float of the
// offset code u = q + 8, then fma(u, s, -8 s), -8 s being exact).  With D
// transposed, a lane ends with four consecutive outputs of one row, which
// the epilogue stores together.
//
// Two kernels, chosen by tile count:
//   gemm_kernel<ACT, MB>: 16 MB x 256 tiles (MB = 8: 128 rows; MB = 4: 64
//     rows for short K), four waves (two workgroups per CU); wave w owns 64
//     columns and all the rows, and dequantizes its own chunks in registers
//     between its MFMAs.
//   gemm8_kernel: 256 x 256 tiles, eight waves (two per SIMD); the
//     workgroup dequantizes each weight once into an LDS operand tile that
//     all waves read, so each weight is decoded once per 256 rows.
// Both stage x in LDS by direct-to-LDS buffer loads (rows past M fall
// outside the buffer and fetch nothing), double-buffered with one barrier
// per stage, and spread the next stage's loads and dequantization between
// the MFMAs of the current one.  Accumulators live in AGPRs (inline-asm
// MFMA with an "a" constraint).
//
// INT8 weights (W8A16) run on gemm8_kernel only: the same stages with a
// 16-byte run of each 1 KB chunk half per stage (byte codes, u = q + 128,
// fma(u, s, -128 s)).
//
// The epilogue adds the bias in FP32 and rounds once to the output dtype, or,
// for a K split, stores FP32 partial sums for the split-K reduce kernel.
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
    float* partials;  // [splits][m][ntiles*256] when splits > 1
    int splits, gps;
    int vec_store;    // y 8-byte aligned and ldy % 4 == 0: 4 outputs per store
    int vec16;        // y 16-byte aligned and ldy % 8 == 0: 8 outputs per store
    int64_t mtiles, ntiles;
};

constexpr int kGmBN = 256, kGmThreads = 256;  // rows per workgroup: 16 * MB
#ifndef GM_PREFETCH
#define GM_PREFETCH 2
#endif
constexpr int kGmPrefetch = GM_PREFETCH;  // A fragments read ahead of their MFMAs

template <int ACT>
__device__ inline void gm_mfma_acc(uint4 a, uint4 b, f32x4_t& c) {
    // accumulator pinned to AGPRs; the two wait states cover a VALU write of
    // an operand just before
    if constexpr (ACT == kActBf16)
        asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
            : "+a"(c)
            : "v"(__builtin_bit_cast(bf16x8_t, a)), "v"(__builtin_bit_cast(bf16x8_t, b)));
    else
        asm("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
            : "+a"(c)
            : "v"(__builtin_bit_cast(f16x8_t, a)), "v"(__builtin_bit_cast(f16x8_t, b)));
}

template <int ACT>
__device__ inline f32x4_t gm_mfma(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (ACT == kActBf16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// Bias of the four output columns c0 .. c0 + 3 of each of a lane's four
// 16-column tiles (t0 .. t0 + 3), in FP32, zero past n or without a bias.
// The sixteen loads use clamped indices and no branches, so all of them are
// in flight together (element-wise conditional loads were each waited for
// before the next was issued).
template <int ACT>
__device__ inline void bias16(const uint16_t* bias, int64_t t0, int kq, int64_t n, float (&bv)[4][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[j][e] = 0.0f;
    if (!bias) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
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

// LDS layout of an x tile: row r of BM rows holds its 128 columns as 16
// segments of 16 bytes, segment c stored at position c ^ (r & 15).  The 16
// lanes of an A-operand read (rows r0..r0+15, one segment each) then touch 16
// different bank groups, with no padding, so each 1 KB piece of the tile can
// be filled by one global_load_lds_dwordx4 (lane i -> LDS bytes 16i..16i+15).
__device__ inline int swz(int row, int seg) { return row * 128 + ((seg ^ (row & 15)) << 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A wave's four 1 KB weight chunks of one group and their dequantization
// into MFMA B operands, one k-step (one word per lane per chunk) at a time.
template <int ACT>
struct GroupWords {
    uint4 w[4];      // this lane's 16 bytes of each chunk: word s = k-step s
    float s[4], o[4];  // scale and -8 * scale per chunk
};

template <int ACT, int MB>
__global__ __launch_bounds__(kGmThreads, MB <= 8 ? 2 : 1) void gemm_kernel(GemmArgs a) {
    constexpr int BM = 16 * MB;
    constexpr int DMA = BM * kGroup * 2 / 1024 / 4;  // 1 KB x pieces per wave per group
    constexpr int NF = 4 * MB;                       // A fragments per wave per group
    __shared__ __align__(16) uint16_t As0[BM * kGroup];
    __shared__ __align__(16) uint16_t As1[BM * kGroup];
    __shared__ __align__(16) uint8_t Bs[16 * kChunkBytes];  // wave w: chunks 4w .. 4w+3

    const Layout L(a.n, a.k);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t tile = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t mt = tile % a.mtiles, nt = tile / a.mtiles;  // consecutive workgroups share weights
    const int64_t m0 = mt * BM;
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;

    // x rows m0 .. m0 + BM - 1 through a buffer resource whose size ends at
    // row M: loads of rows past M are out of range and fetch nothing (those
    // rows only feed outputs that are never stored).  Piece p of a wave
    // covers tile rows 4 * (wave * DMA + p) .. +3; lane i lands at row
    // + i / 16, position i % 16, which holds segment (i % 16) ^ (row & 15).
    // Row & 15 repeats every four pieces, so four lane offsets serve all.
    const int64_t rows_valid = min<int64_t>(BM, a.m - m0);
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(a.x + m0 * a.ldx, rows_valid * a.ldx * 2);
    uint32_t xoff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = wave * DMA * 4 + 4 * p + (lane >> 4);
        xoff[p] = uint32_t(row * a.ldx * 2 + (((lane & 15) ^ (row & 15)) << 4));
    }
    const uint32_t xstep16 = uint32_t(16 * a.ldx * 2);  // 16 rows
    auto load_x_piece = [&](uint16_t* dst, int64_t g, int p) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_ptr_t)(dst + (wave * DMA + p) * 512), 16,
                                                 xoff[p & 3] + uint32_t(p >> 2) * xstep16,
                                                 uniform(int(g * kGroup * 2)), 0, 0);
    };

    // This wave's four row tiles t0 + j (j = 0..3) are consecutive, so their
    // chunks of a group are kGroups * 1 KB apart.  Tiles past N read the last
    // tile again (clamped); their scales are zeroed and outputs never stored.
    // A chunk is exactly the lane-ordered 1 KB a wave's 16-byte direct load
    // writes, so lane L later reads back its own 16 bytes; scales go to
    // registers.
    const int64_t t0 = nt * 16 + wave * 4;
    const int valid = int(min<int64_t>(4, max<int64_t>(0, L.tiles - t0)));
    const int64_t tfirst = min<int64_t>(t0, L.tiles - 1);
    const __amdgpu_buffer_rsrc_t wres =
        buffer_rsrc(a.packed + tfirst * L.groups * kChunkBytes, 4 * L.groups * kChunkBytes);
    const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(
        a.packed + L.scale_offset() + tfirst * L.groups * kChunkScaleBytes, 4 * L.groups * kChunkScaleBytes);
    uint32_t woff[4], soff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int jj = j < valid ? j : (valid > 0 ? valid - 1 : 0);
        woff[j] = uint32_t(jj * L.groups * kChunkBytes + lane * 16);
        soff[j] = uint32_t(jj * L.groups * kChunkScaleBytes + r * 4);
    }
    float sc[4];
    auto load_w_chunk = [&](int64_t g, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_ptr_t)(Bs + (wave * 4 + j) * kChunkBytes), 16,
                                                 woff[j], uniform(int(g * kChunkBytes)), 0, 0);
        sc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              sres, soff[j], uniform(int(g * kChunkScaleBytes)), 0));
    };
    // this wave's chunk words and scales of a group, once its loads landed
    auto take_words = [&](GroupWords<ACT>& gw) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gw.w[j] = *reinterpret_cast<const uint4*>(Bs + (wave * 4 + j) * kChunkBytes + lane * 16);
            gw.s[j] = j < valid ? sc[j] : 0.0f;
            gw.o[j] = -8.0f * gw.s[j];
        }
    };

    f32x4_t acc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One group, software-pipelined.  On entry the group's x tile sits in A
    // (after the barrier below), its chunk words in cur and k-step 0's B
    // operands in bc.  The four k-steps run as MB blocks each: four MFMAs on
    // one A fragment (read two blocks ahead) plus one slice of other work,
    // fenced so that the slices stay spread between the MFMAs:
    //   k-step 0: one of the next group's x pieces into Anext;
    //   k-step 1: one of its weight chunks and scales (blocks 0..3);
    //   k-steps 0..2: a quarter word of the next k-step's B operands;
    //   k-step 3: once the next group's chunks landed, a quarter word of its
    //             k-step 0 B operands.
    // The two x buffers keep fixed roles in each half of the unrolled pair
    // below so the compiler can tell the direct loads into Anext from the
    // reads of A.
    GroupWords<ACT> cur, nxt;
    uint4 bc[4], bn[4];
    auto group = [&](const uint16_t* A, uint16_t* Anext, int gl) {
        __builtin_amdgcn_s_barrier();  // every wave's x pieces of this group landed
        const bool more = gl + 1 < ng;
        const int64_t gn = g0 + gl + 1;
        uint4 af[kGmPrefetch + 1];
        auto read_a = [&](int f) {
            const int sk = f / MB, i = f % MB;
            return *reinterpret_cast<const uint4*>(A + swz(i * 16 + r, 4 * sk + kq));
        };
#pragma unroll
        for (int f = 0; f < kGmPrefetch; ++f) af[f] = read_a(f);
#pragma unroll
        for (int sk = 0; sk < 4; ++sk) {
            if (sk == 3 && more) {
                // the next group's chunks, scales and x pieces were issued
                // two k-steps ago
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                take_words(nxt);
            }
            // dequantization temporaries carried between the quarter slices
            uint32_t lo = 0, hi = 0;
            float c0 = 0.f, c4 = 0.f, c2 = 0.f, c6 = 0.f;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int f = sk * MB + i;
                const uint4 aop = af[f % (kGmPrefetch + 1)];
                if (f + kGmPrefetch < NF) af[(f + kGmPrefetch) % (kGmPrefetch + 1)] = read_a(f + kGmPrefetch);
                if (sk == 0 && i < DMA && more) load_x_piece(Anext, gn, i);
                if (sk == 1 && i < 4 && more) load_w_chunk(gn, i);
#pragma unroll
                for (int j = 0; j < 4; ++j) gm_mfma_acc<ACT>(bc[j], aop, acc[i][j]);
                // word j of the next k-step (k-step 3: the next group's
                // k-step 0) in MB / 4 slices, quarters q0 .. q0 + 4 / PER - 1
                constexpr int PER = MB / 4;
                const int j = i / PER, q0 = (i % PER) * (4 / PER);
                if (sk < 3 || more) {
                    const GroupWords<ACT>& src = sk < 3 ? cur : nxt;
                    const uint32_t w = sk == 0 ? src.w[j].y : sk == 1 ? src.w[j].z : sk == 2 ? src.w[j].w : src.w[j].x;
                    const float sj = src.s[j], oj = src.o[j];
#pragma unroll
                    for (int q = q0; q < q0 + 4 / PER; ++q) {
                        if (q == 0) {
                            lo = w & 0x0F0F0F0Fu;  // bytes: columns 0, 4, 1, 5
                            c0 = fmaf(byte_f32<0>(lo), sj, oj);
                            c4 = fmaf(byte_f32<1>(lo), sj, oj);
                        } else if (q == 1) {
                            const float c1 = fmaf(byte_f32<2>(lo), sj, oj);
                            const float c5 = fmaf(byte_f32<3>(lo), sj, oj);
                            bn[j].x = pack2<ACT>(c0, c1);
                            bn[j].z = pack2<ACT>(c4, c5);
                        } else if (q == 2) {
                            hi = (w >> 4) & 0x0F0F0F0Fu;  // bytes: columns 2, 6, 3, 7
                            c2 = fmaf(byte_f32<0>(hi), sj, oj);
                            c6 = fmaf(byte_f32<1>(hi), sj, oj);
                        } else {
                            const float c3 = fmaf(byte_f32<2>(hi), sj, oj);
                            const float c7 = fmaf(byte_f32<3>(hi), sj, oj);
                            bn[j].y = pack2<ACT>(c2, c3);
                            bn[j].w = pack2<ACT>(c6, c7);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) bc[j] = bn[j];
        }
        cur = nxt;
    };

    // prologue: group g0's loads, its words and k-step 0 operands
#pragma unroll
    for (int p = 0; p < DMA; ++p) load_x_piece(As0, g0, p);
#pragma unroll
    for (int j = 0; j < 4; ++j) load_w_chunk(g0, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    take_words(cur);
#pragma unroll
    for (int j = 0; j < 4; ++j) bc[j] = dequant_word<ACT>(cur.w[j].x, cur.s[j], cur.o[j]);
    // Bs is refilled (next group's chunks) only after every word was read
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    int gl = 0;
    for (; gl + 1 < ng; gl += 2) {
        group(As0, As1, gl);
        group(As1, As0, gl + 1);
    }
    if (gl < ng) group(As0, As1, gl);
    // results of the last MFMAs are read by ordinary instructions below:
    // wait out the pipeline first, then mark every accumulator as produced
    // after the wait
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));

    // --- epilogue.  Each 16 x 16 block is D = W . x^T: lane (r, kq) holds
    // outputs 4kq .. 4kq + 3 of tile t0 + j for x row r of row block i, four
    // consecutive columns (one 8-byte store, 16 bytes for FP32 partials).
    const int64_t npad = a.ntiles * kGmBN;
    float ball[4][4];
    bias16<ACT>(a.splits == 1 ? a.bias : nullptr, t0, kq, a.n, ball);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t c0 = (t0 + j) * 16 + 4 * kq;
        if (c0 >= a.n) continue;
        const bool full = c0 + 4 <= a.n;
        const float* bv = ball[j];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int64_t row = m0 + i * 16 + r;
            if (row >= a.m) continue;
            const f32x4_t v = acc[i][j];
            if (a.splits > 1) {
                *reinterpret_cast<f32x4_t*>(a.partials + (int64_t(split) * a.m + row) * npad + c0) = v;
            } else if (full && a.vec_store) {
                *reinterpret_cast<uint2*>(a.y + row * a.ldy + c0) =
                    make_uint2(pack2<ACT>(v[0] + bv[0], v[1] + bv[1]), pack2<ACT>(v[2] + bv[2], v[3] + bv[3]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < a.n) a.y[row * a.ldy + c0 + e] = from_f32<ACT>(v[e] + bv[e]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Eight-wave variant: a 256 x 256 output tile per workgroup, two waves per
// SIMD, each wave 128 rows x 64 columns (128 accumulators).  The K loop runs
// in stages of 64 (half a quantization group).  Per stage the workgroup
// stages in LDS the x tile (256 rows x 64, by direct loads) and the B tile:
// the stage's weights dequantized to 16-bit MFMA operands, 16 tiles x 2
// k-steps x 64 lanes x 16 bytes.  Each wave dequantizes two of the 16 weight
// tiles (one word per lane per k-step, written where the reading lane finds
// it), so each weight is dequantized once per 256 rows of x while every wave
// keeps only 128 accumulators.
// ---------------------------------------------------------------------------
template <bool B>
struct BoolC {
    static constexpr bool value = B;
};
constexpr int kG8Threads = 512, kG8Rows = 256, kG8K = 64;
constexpr int kG8XStage = kG8Rows * kG8K;          // 16-bit elements per x stage
constexpr int kG8WStage = 16 * 2 * 64 * 16;        // bytes per B stage

// x stage layout: row r holds its 64 columns as 8 segments of 16 bytes,
// segment c at position c ^ ((r >> 1) & 7): the 16 lanes of an operand read
// (16 consecutive rows, one segment) cover all 64 banks once.
__device__ inline int swz8(int row, int seg) { return row * kG8K + ((seg ^ ((row >> 1) & 7)) << 3); }

// BITS 8: INT8 chunks (two 1 KB halves, half h = stage 2g + h): a lane's
// k-step is two words of four byte codes, u = q + 128.
template <int ACT, bool STAGED, int BITS>
__global__ __launch_bounds__(kG8Threads, 1) void gemm8_kernel(GemmArgs a) {
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    __shared__ __align__(16) uint16_t X0[kG8XStage];
    __shared__ __align__(16) uint16_t X1[kG8XStage];
    __shared__ __align__(16) uint8_t W0[kG8WStage];
    __shared__ __align__(16) uint8_t W1[kG8WStage];

    const Layout L(a.n, a.k, BITS);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t tile = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t mt = tile % a.mtiles, nt = tile / a.mtiles;  // consecutive workgroups share weights
    const int64_t m0 = mt * kG8Rows;
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));
    const int nstages = 2 * ng;

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int wm = wave >> 2, wn = wave & 3;  // 128-row half, 64-column quarter

    // x: rows m0 .. m0 + 255 through a buffer resource ending at row M (loads
    // of rows past M fetch nothing; those rows only feed outputs never
    // stored).  Piece p of wave w fills stage rows 8 (4w + p) .. +7; lane i
    // lands at row + i / 8, position i % 8.
    const int64_t rows_valid = min<int64_t>(kG8Rows, a.m - m0);
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(a.x + m0 * a.ldx, rows_valid * a.ldx * 2);
    uint32_t xoff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = 8 * (4 * wave + p) + (lane >> 3);
        xoff[p] = uint32_t(row * a.ldx * 2 + (((lane & 7) ^ ((row >> 1) & 7)) << 4));
    }
    auto load_x = [&](uint16_t* dst, int s) {
        const int soff = uniform(int((g0 + (s >> 1)) * kGroup * 2 + (s & 1) * kG8K * 2));
#pragma unroll
        for (int p = 0; p < 4; ++p)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_ptr_t)(dst + (4 * wave + p) * 512), 16, xoff[p],
                                                     soff, 0, 0);
    };

    // Weights: this wave dequantizes the workgroup's tiles 2w and 2w + 1.
    // Tiles past N read the last tile again (clamped) with their scales
    // zeroed.
    const int64_t tw = nt * 16 + 2 * wave;
    const int validw = int(min<int64_t>(2, max<int64_t>(0, L.tiles - tw)));
    const int64_t twfirst = min<int64_t>(tw, L.tiles - 1);
    const __amdgpu_buffer_rsrc_t wres =
        buffer_rsrc(a.packed + twfirst * L.groups * CB, 2 * L.groups * CB);
    const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(
        a.packed + L.scale_offset() + twfirst * L.groups * kChunkScaleBytes, 2 * L.groups * kChunkScaleBytes);
    uint32_t woff[2], soff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int cc = c < validw ? c : (validw > 0 ? validw - 1 : 0);
        woff[c] = uint32_t(cc * L.groups * CB + lane * 16);
        soff[c] = uint32_t(cc * L.groups * kChunkScaleBytes + r * 4);
    }
    struct Words {
        uint32_t w[2][4 * H];  // INT8: half h in words 4h .. 4h + 3
        float s[2];
    };
    // one group's words and scales (groups past the split's end reload its
    // last group, keeping the count of loads in flight fixed)
    auto load_words = [&](Words& d, int gl) {
        const int64_t g = g0 + min(gl, ng - 1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[c] + h * kChunkBytes,
                                                                     uniform(int(g * CB)), 0);
                d.w[c][4 * h] = v[0];
                d.w[c][4 * h + 1] = v[1];
                d.w[c][4 * h + 2] = v[2];
                d.w[c][4 * h + 3] = v[3];
            }
            d.s[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   sres, soff[c], uniform(int(g * kChunkScaleBytes)), 0));
        }
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    Words wcur, wnext, wfut;
    // B-stage slot of (tile, k-step) for this lane
    auto wslot = [&](int tt, int ks) { return ((tt * 2 + ks) * 64 + lane) * 16; };

    // One stage: wait for its x pieces and B tile, barrier, start the next
    // stage's x loads (and at a group's first stage the weight words two
    // groups ahead), then 16 blocks of four MFMAs, each with a quarter word
    // of the next stage's dequantization; a finished word goes to the next
    // B tile.  Fixed buffer roles per call let the compiler tell the direct
    // loads and B writes into the next stage from the reads of this one.
    // The last stage also loads and dequantizes (its own x and B again, into
    // buffers nobody reads any more), which keeps the loop free of branches.
    auto stage = [&](const uint16_t* Xp, const uint8_t* Wp, uint16_t* Xq, uint8_t* Wq, int s, auto odd_c) {
        constexpr bool odd = decltype(odd_c)::value;
        // an even stage issued its successor's x pieces and then the word
        // loads (two 16-byte runs and two scales; INT8: four runs); an odd
        // stage only x pieces
        if constexpr (odd && BITS == 8)
            asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)" ::: "memory");
        else if constexpr (odd)
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        load_x(Xq, min(s + 1, nstages - 1));
        if constexpr (!odd) load_words(wfut, (s >> 1) + 2);
        // words of stage s + 1: the second half of this group, or the first
        // half of the next
        const Words& src = odd ? wnext : wcur;
        constexpr int h1 = odd ? 0 : 1;

        uint4 xf[3];
        auto read_x = [&](int f) {
            const int ks = f >> 3, i = f & 7;
            return *reinterpret_cast<const uint4*>(Xp + swz8(wm * 128 + i * 16 + r, 4 * ks + kq));
        };
        xf[0] = read_x(0);
        xf[1] = read_x(1);
        uint4 wf[4];
        uint32_t lo = 0, hi = 0;
        float c0 = 0.f, c4 = 0.f, c2 = 0.f, c6 = 0.f;
        uint4 out = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            const int ks = f >> 3, i = f & 7;
            if (i == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    wf[j] = *reinterpret_cast<const uint4*>(Wp + wslot(wn * 4 + j, ks));
            }
            const uint4 xop = xf[f % 3];
            if (f + 2 < 16) xf[(f + 2) % 3] = read_x(f + 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) gm_mfma_acc<ACT>(wf[j], xop, acc[i][j]);
            {
                // word (c, ks') of stage s + 1: c = f / 8, ks' = (f / 4) % 2,
                // quarter f % 4
                const int c = f >> 3, kn = (f >> 2) & 1, q = f & 3;
                const float sj = c < validw ? src.s[c] : 0.0f;
                if constexpr (BITS == 8) {
                    // words 4 h1 + 2 kn (columns 0-3) and + 1 (columns 4-7):
                    // quarter q converts columns 2q, 2q + 1
                    const uint32_t w = src.w[c][4 * h1 + 2 * kn + (q >> 1)];
                    const float oj = -128.0f * sj;
                    const float va = fmaf((q & 1) ? byte_f32<2>(w) : byte_f32<0>(w), sj, oj);
                    const float vb = fmaf((q & 1) ? byte_f32<3>(w) : byte_f32<1>(w), sj, oj);
                    const uint32_t pr = pack2<ACT>(va, vb);
                    if (q == 0) out.x = pr;
                    else if (q == 1) out.y = pr;
                    else if (q == 2) out.z = pr;
                    else {
                        out.w = pr;
                        *reinterpret_cast<uint4*>(Wq + wslot(2 * wave + c, kn)) = out;
                    }
                } else {
                const uint32_t w = src.w[c][2 * h1 + kn];
                const float oj = -8.0f * sj;
                if (q == 0) {
                    lo = w & 0x0F0F0F0Fu;  // bytes: columns 0, 4, 1, 5
                    c0 = fmaf(byte_f32<0>(lo), sj, oj);
                    c4 = fmaf(byte_f32<1>(lo), sj, oj);
                } else if (q == 1) {
                    const float c1 = fmaf(byte_f32<2>(lo), sj, oj);
                    const float c5 = fmaf(byte_f32<3>(lo), sj, oj);
                    out.x = pack2<ACT>(c0, c1);
                    out.z = pack2<ACT>(c4, c5);
                } else if (q == 2) {
                    hi = (w >> 4) & 0x0F0F0F0Fu;  // bytes: columns 2, 6, 3, 7
                    c2 = fmaf(byte_f32<0>(hi), sj, oj);
                    c6 = fmaf(byte_f32<1>(hi), sj, oj);
                } else {
                    const float c3 = fmaf(byte_f32<2>(hi), sj, oj);
                    const float c7 = fmaf(byte_f32<3>(hi), sj, oj);
                    out.y = pack2<ACT>(c2, c3);
                    out.w = pack2<ACT>(c6, c7);
                    *reinterpret_cast<uint4*>(Wq + wslot(2 * wave + c, kn)) = out;
                }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (odd) {
            wcur = wnext;
            wnext = wfut;
        }
    };

    // prologue: stage 0's x, the first two groups' words, stage 0's B tile
    load_x(X0, 0);
    load_words(wcur, 0);
    load_words(wnext, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float sj = c < validw ? wcur.s[c] : 0.0f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            *reinterpret_cast<uint4*>(W0 + wslot(2 * wave + c, ks)) =
                BITS == 8 ? dequant_word8<ACT>(wcur.w[c][2 * ks], wcur.w[c][2 * ks + 1], sj, -128.0f * sj)
                          : dequant_word<ACT>(wcur.w[c][ks], sj, -8.0f * sj);
    }

    for (int s = 0; s < nstages; s += 2) {
        stage(X0, W0, X1, W1, s, BoolC<false>{});
        stage(X1, W1, X0, W0, s + 1, BoolC<true>{});
    }
    // results of the last MFMAs are read by ordinary instructions below:
    // wait out the pipeline first, then mark every accumulator as produced
    // after the wait
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));

    // --- epilogue: lane (r, kq) holds outputs 4kq .. 4kq + 3 of tile t0 + j
    // for x row r of row block i
    const int64_t npad = a.ntiles * kGmBN;
    const int64_t t0 = nt * 16 + wn * 4;
    if constexpr (STAGED) {
        // Through LDS (one K split, 16-byte aligned rows): the 256 x 256 tile of 16-bit outputs (512 bytes a row)
        // fills the four stage buffers, 64 rows each, and leaves as whole
        // rows in 16-byte stores.  Within a row, 16-byte unit u sits at
        // position u ^ (row & 31), so the sixteen rows one write touches and
        // the 32 units one row read touches spread over all banks.
        __builtin_amdgcn_s_barrier();  // every wave is done with the last stage
        auto tile_row = [&](int row) -> uint8_t* {
            uint8_t* q = (row >> 6) == 0   ? reinterpret_cast<uint8_t*>(X0)
                         : (row >> 6) == 1 ? reinterpret_cast<uint8_t*>(X1)
                         : (row >> 6) == 2 ? W0
                                           : W1;
            return q + (row & 63) * 512;
        };
        float ball[4][4];
        bias16<ACT>(a.bias, t0, kq, a.n, ball);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float* bv = ball[j];
            const int u = (wn * 4 + j) * 2 + (kq >> 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = wm * 128 + i * 16 + r;
                const f32x4_t v = acc[i][j];
                *reinterpret_cast<uint2*>(tile_row(row) + ((u ^ (row & 31)) << 4) + (kq & 1) * 8) =
                    make_uint2(pack2<ACT>(v[0] + bv[0], v[1] + bv[1]), pack2<ACT>(v[2] + bv[2], v[3] + bv[3]));
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        const int u = tid & 31;
        const int64_t col = nt * kGmBN + u * 8;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = it * 16 + (tid >> 5);
            const int64_t grow = m0 + row;
            const uint4 v = *reinterpret_cast<const uint4*>(tile_row(row) + ((u ^ (row & 31)) << 4));
            if (grow >= a.m || col >= a.n) continue;
            uint16_t* dst = a.y + grow * a.ldy + col;
            if (col + 8 <= a.n) {
                *reinterpret_cast<uint4*>(dst) = v;
            } else {
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                for (int e = 0; e < 8 && col + e < a.n; ++e) dst[e] = uint16_t(w4[e >> 1] >> (16 * (e & 1)));
            }
        }
    } else {
    float ball[4][4];
    bias16<ACT>(a.splits == 1 ? a.bias : nullptr, t0, kq, a.n, ball);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t c0 = (t0 + j) * 16 + 4 * kq;
        if (c0 >= a.n) continue;
        const bool full = c0 + 4 <= a.n;
        const float* bv = ball[j];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = m0 + wm * 128 + i * 16 + r;
            if (row >= a.m) continue;
            const f32x4_t v = acc[i][j];
            if (a.splits > 1) {
                *reinterpret_cast<f32x4_t*>(a.partials + (int64_t(split) * a.m + row) * npad + c0) = v;
            } else if (full && a.vec_store) {
                *reinterpret_cast<uint2*>(a.y + row * a.ldy + c0) =
                    make_uint2(pack2<ACT>(v[0] + bv[0], v[1] + bv[1]), pack2<ACT>(v[2] + bv[2], v[3] + bv[3]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < a.n) a.y[row * a.ldy + c0 + e] = from_f32<ACT>(v[e] + bv[e]);
            }
        }
    }
    }
}

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, int bits) {
    GemmPlan p{};
    const Layout L(n, k, bits);
    // 256 x 256 tiles (eight waves, each weight dequantized once per 256
    // rows) where they alone give every CU work; else 128 x 256 tiles of
    // four waves, two workgroups per CU.
    // Also where a K split leaves each 256 x 256 part at least 16 groups
    // (long K: 1024 x 2048 x 16384 took 80.9 us in eight parts of 256 x 256
    // against 84.1 us in four of 128 x 256).
    const int64_t tiles8 = ceil_div(m, kG8Rows) * ceil_div(n, kGmBN);
    const int64_t splits8 = tiles8 >= 256 ? 1 : 256 / tiles8;
    p.waves = tiles8 >= 128 || L.groups >= 16 * splits8 ? 8 : 4;
    if (bits == 8) p.waves = 8;  // INT8 weights: the eight-wave kernel only
    p.mb = p.waves == 8 ? 16 : 8;
    // A short K (<= 16 groups) whose 128-row tiles would need a K split takes
    // 64-row tiles: twice the workgroups, and no partial sums to write and
    // reduce (1024 x 4096 x 1024: 31.5 -> 19.7 us; 256 x 16384 x 2048: 37.2
    // -> 33.9 us).  Up to 8 groups it never splits; with more, tiles filling
    // half the chip split in two (100 x 16384 x 2048: 25.7 us against 31.4
    // unsplit).
    const bool rows64 = p.waves == 4 && L.groups <= 16 && ceil_div(m, 128) * ceil_div(n, kGmBN) < 256;
    if (rows64) p.mb = 4;
    p.mtiles = ceil_div(m, 16 * p.mb);
    p.ntiles = ceil_div(n, kGmBN);
    const int64_t tiles = p.mtiles * p.ntiles;
    // split K while the tiles alone leave CUs idle, into as many parts as
    // still fit one round of 256 workgroups (a second, partial round would
    // cost a whole round's time)
    int64_t splits = tiles >= 256 ? 1 : 256 / tiles;
    if (rows64 && L.groups <= 8) splits = 1;
    if (splits > L.groups) splits = L.groups;
    int64_t gps = ceil_div(L.groups, splits);
    p.gps = int(gps);
    p.splits = int(ceil_div(L.groups, gps));
    p.workspace = p.splits > 1 ? kSyncBytes + size_t(p.splits) * m * p.ntiles * kGmBN * 4 : 0;
    return p;
}

template <int BITS>
static void launch_g8(const GemmArgs& a, bool bf, bool staged, dim3 grid, hipStream_t stream) {
    const dim3 b8(kG8Threads);
    if (staged) {
        if (bf) gemm8_kernel<kActBf16, true, BITS><<<grid, b8, 0, stream>>>(a);
        else gemm8_kernel<kActF16, true, BITS><<<grid, b8, 0, stream>>>(a);
    } else {
        if (bf) gemm8_kernel<kActBf16, false, BITS><<<grid, b8, 0, stream>>>(a);
        else gemm8_kernel<kActF16, false, BITS><<<grid, b8, 0, stream>>>(a);
    }
}

hipError_t launch_gemm(const void* x, int act, int bits, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream) {
    const GemmPlan p = plan_gemm(m, n, k, bits);
    // the x tile's buffer resource takes 32-bit byte offsets
    if (int64_t(16 * p.mb) * ldx * 2 > int64_t(0xFFFFFFFF)) return hipErrorInvalidValue;
    GemmArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.m = m;
    a.packed = static_cast<const uint8_t*>(packed);
    a.n = n;
    a.k = k;
    a.bias = static_cast<const uint16_t*>(bias);
    a.y = static_cast<uint16_t*>(y);
    a.ldy = ldy;
    a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSyncBytes);
    a.vec_store = reinterpret_cast<uintptr_t>(y) % 8 == 0 && ldy % 4 == 0;
    a.vec16 = reinterpret_cast<uintptr_t>(y) % 16 == 0 && ldy % 8 == 0;
    a.splits = p.splits;
    a.gps = p.gps;
    a.mtiles = p.mtiles;
    a.ntiles = p.ntiles;
    const dim3 grid(unsigned(p.mtiles * p.ntiles * p.splits)), block(kGmThreads);
    const bool bf = act == kActBf16;
    if (p.waves == 8) {
        if (bits == 8) launch_g8<8>(a, bf, p.splits == 1 && a.vec16, grid, stream);
        else launch_g8<4>(a, bf, p.splits == 1 && a.vec16, grid, stream);
    } else {
        if (p.mb == 4) {
            if (bf) gemm_kernel<kActBf16, 4><<<grid, block, 0, stream>>>(a);
            else gemm_kernel<kActF16, 4><<<grid, block, 0, stream>>>(a);
        } else {
            if (bf) gemm_kernel<kActBf16, 8><<<grid, block, 0, stream>>>(a);
            else gemm_kernel<kActF16, 8><<<grid, block, 0, stream>>>(a);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(a.partials, p.splits, m, n, p.ntiles * kGmBN, a.bias, a.y, a.ldy, act, stream);
}

}  // namespace w4a16
