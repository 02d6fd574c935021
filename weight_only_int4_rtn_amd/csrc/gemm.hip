// Large-M forward: the layer as a dense contraction on the matrix cores.
//
// A workgroup of 4 waves computes a BM x 256 tile of y; wave w owns the 64
// columns of row tiles 4w .. 4w+3 and all BM rows (BM / 16 blocks of
// v_mfma_f32_16x16x32_{bf16,f16} per column tile).  K advances one
// 128-column scale group per iteration.
//
// Weights never pass through LDS: the packed chunk is the MFMA B-operand
// layout (lane L: column L % 16 of the tile, columns 8*(L/16) + j of each
// 32-wide k-step), so each wave loads its four chunks with one 128-bit load
// per lane each and dequantizes them in registers as q * s rounded once to
// the 16-bit input type (byte -> float of the offset code u = q + 8, then
// fma(u, s, -8 s), -8 s being exact).  The x tile is shared by the 4 waves
// through LDS, double-buffered: while the waves run the MFMAs of group g, the
// loads of group g + 1 (x rows and weight chunks) are in flight, so one
// barrier per group suffices.  LDS rows are padded by 16 bytes against bank
// conflicts.
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
    float* partials;  // [splits][m][ntiles*128] when splits > 1
    int splits, gps;
    int64_t mtiles, ntiles;
};

constexpr int kGmBN = 256, kGmThreads = 256;  // rows per workgroup: 16 * MB

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

// LDS layout of an x tile: row r of BM rows holds its 128 columns as 16
// segments of 16 bytes, segment c stored at position c ^ (r & 15).  The 16
// lanes of an A-operand read (rows r0..r0+15, one segment each) then touch 16
// different bank groups, with no padding, so each 1 KB piece of the tile can
// be filled by one global_load_lds_dwordx4 (lane i -> LDS bytes 16i..16i+15).
__device__ inline int swz(int row, int seg) { return row * 128 + ((seg ^ (row & 15)) << 3); }

template <int ACT, int MB>
__global__ __launch_bounds__(kGmThreads, MB <= 8 ? 2 : 1) void gemm_kernel(GemmArgs a) {
    constexpr int BM = 16 * MB;
    constexpr int DMA = BM * kGroup * 2 / 1024 / 4;  // 1 KB direct loads per wave per group
    __shared__ __align__(16) uint16_t As0[BM * kGroup];
    __shared__ __align__(16) uint16_t As1[BM * kGroup];

    const Layout L(a.n, a.k);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t tile = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t mt = tile % a.mtiles, nt = tile / a.mtiles;  // consecutive workgroups share weights
    const int64_t m0 = mt * BM;
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const float* scales = reinterpret_cast<const float*>(a.packed + L.scale_offset());

    // This wave's four row tiles t0 + j (j = 0..3) are consecutive, so their
    // chunks of a group are kGroups * 1 KB apart.  Tiles past N are clamped to
    // the last one; their outputs are never stored.
    const int64_t t0 = nt * 16 + wave * 4;
    const int64_t tile_step = L.groups * kChunkBytes;
    const uint8_t* cbase = a.packed + (min<int64_t>(t0, L.tiles - 1) * L.groups) * kChunkBytes + lane * 16;
    const float* sbase = scales + min<int64_t>(t0, L.tiles - 1) * L.groups * kTileRows + r;
    const int valid = int(min<int64_t>(4, max<int64_t>(0, L.tiles - t0)));  // tiles of this wave inside N

    // Direct x loads: piece p covers tile rows 4 * (wave * DMA + p) .. +3;
    // lane i lands at row + i / 16, position i % 16, which holds segment
    // (i % 16) ^ (row & 15).  Rows past M are clamped (they feed outputs that
    // are never stored).
    const int drow0 = wave * DMA * 4 + (lane >> 4);
    auto load_x = [&](uint16_t* dst, int64_t g) {
        // recompute the source addresses every group rather than keeping
        // DMA 64-bit pointers live across the loop (they would spill)
        int rbase = drow0;
        asm volatile("" : "+v"(rbase));
#pragma unroll
        for (int p = 0; p < DMA; ++p) {
            const int row = rbase + 4 * p;
            const int seg = (lane & 15) ^ (row & 15);
            const int64_t gr = m0 + row < a.m ? m0 + row : a.m - 1;
            __builtin_amdgcn_global_load_lds(a.x + gr * a.ldx + g * kGroup + seg * 8,
                                             (__attribute__((address_space(3))) void*)(dst + (wave * DMA + p) * 512),
                                             16, 0, 0);
        }
    };
    uint4 cw[4];
    float sc[4];
    auto load_w = [&](int64_t g) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int jj = j < valid ? j : (valid > 0 ? valid - 1 : 0);
            cw[j] = *reinterpret_cast<const uint4*>(cbase + jj * tile_step + g * kChunkBytes);
            sc[j] = sbase[jj * L.groups * kTileRows + g * kTileRows];
        }
    };

    f32x4_t acc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One group: wait for its x pieces and weights, barrier (A complete, and
    // nobody reads Anext any more), start the next group's loads into Anext
    // and registers, then run the MFMAs on A.  The two buffers keep fixed
    // roles in each half of the unrolled pair below, so the compiler can
    // tell the direct loads into Anext from the reads of A.
    auto group = [&](const uint16_t* A, uint16_t* Anext, int gl) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        uint4 cur[4];
        float s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            cur[j] = cw[j];
            s4[j] = j < valid ? sc[j] : 0.0f;
        }
        if (gl + 1 < ng) {
            load_x(Anext, g0 + gl + 1);
            load_w(g0 + gl + 1);
        }
#pragma unroll
        for (int sk = 0; sk < 4; ++sk) {
            uint4 bop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = sk == 0 ? cur[j].x : sk == 1 ? cur[j].y : sk == 2 ? cur[j].z : cur[j].w;
                bop[j] = dequant_word<ACT>(w, s4[j], -8.0f * s4[j]);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const uint4 aop = *reinterpret_cast<const uint4*>(A + swz(i * 16 + r, 4 * sk + kq));
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = gm_mfma<ACT>(aop, bop[j], acc[i][j]);
            }
            // keep each k-step's operands from piling up in registers
            if constexpr (MB > 8) __builtin_amdgcn_sched_barrier(0);
        }
    };

    load_x(As0, g0);
    load_w(g0);
    for (int gl = 0; gl < ng; gl += 2) {
        group(As0, As1, gl);
        if (gl + 1 < ng) group(As1, As0, gl + 1);
    }

    // --- epilogue: lane holds rows 4kq + e of column r of each 16 x 16 block
    const int64_t npad = a.ntiles * kGmBN;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t col = (t0 + j) * 16 + r;
        if (col >= a.n) continue;
        const float bv = (a.splits == 1 && a.bias) ? to_f32<ACT>(a.bias[col]) : 0.0f;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + i * 16 + 4 * kq + e;
                if (row >= a.m) continue;
                if (a.splits == 1)
                    a.y[row * a.ldy + col] = from_f32<ACT>(acc[i][j][e] + bv);
                else
                    a.partials[(int64_t(split) * a.m + row) * npad + col] = acc[i][j][e];
            }
    }
}

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k) {
    GemmPlan p{};
    const Layout L(n, k);
    // 256 rows per workgroup halve the dequantization work per MFMA; 128
    // rows keep two workgroups per CU where M is small.
    p.mb = 8;
    p.mtiles = ceil_div(m, 16 * p.mb);
    p.ntiles = ceil_div(n, kGmBN);
    const int64_t tiles = p.mtiles * p.ntiles;
    // split K while the tiles alone leave CUs idle (aim for >= 256 workgroups)
    int64_t splits = tiles >= 256 ? 1 : ceil_div(256, tiles);
    if (splits > L.groups) splits = L.groups;
    int64_t gps = ceil_div(L.groups, splits);
    p.gps = int(gps);
    p.splits = int(ceil_div(L.groups, gps));
    p.workspace = p.splits > 1 ? size_t(p.splits) * m * p.ntiles * kGmBN * 4 : 0;
    return p;
}

hipError_t launch_gemm(const void* x, int act, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream) {
    const GemmPlan p = plan_gemm(m, n, k);
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
    a.partials = static_cast<float*>(workspace);
    a.splits = p.splits;
    a.gps = p.gps;
    a.mtiles = p.mtiles;
    a.ntiles = p.ntiles;
    const dim3 grid(unsigned(p.mtiles * p.ntiles * p.splits)), block(kGmThreads);
    const bool bf = act == kActBf16;
    if (p.mb == 16) {
        if (bf) gemm_kernel<kActBf16, 16><<<grid, block, 0, stream>>>(a);
        else gemm_kernel<kActF16, 16><<<grid, block, 0, stream>>>(a);
    } else if (p.mb == 12) {
        if (bf) gemm_kernel<kActBf16, 12><<<grid, block, 0, stream>>>(a);
        else gemm_kernel<kActF16, 12><<<grid, block, 0, stream>>>(a);
    } else {
        if (bf) gemm_kernel<kActBf16, 8><<<grid, block, 0, stream>>>(a);
        else gemm_kernel<kActF16, 8><<<grid, block, 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(a.partials, p.splits, m, n, p.ntiles * kGmBN, a.bias, a.y, a.ldy, act, stream);
}

}  // namespace w4a16
