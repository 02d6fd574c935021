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

constexpr int kGmBM = 128, kGmBN = 256, kGmThreads = 256;
constexpr int kGmStride = kGroup + 8;  // LDS row stride (elements)

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

// Two FP32 values -> packed pair of the 16-bit type (round to nearest even).
template <int ACT>
__device__ inline uint32_t pack2(float lo, float hi) {
    return uint32_t(from_f32<ACT>(lo)) | (uint32_t(from_f32<ACT>(hi)) << 16);
}

// Byte B of a word as a float (selected as v_cvt_f32_ubyteB).
template <int B>
__device__ inline float byte_f32(uint32_t w) {
    return float((w >> (8 * B)) & 0xFFu);
}

// One packed word (8 codes of columns j = 0..7, nibble i = column 2i, nibble
// i + 4 = column 2i + 1) -> 8 dequantized 16-bit values in column order.
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

template <int ACT, int MB>
__global__ __launch_bounds__(kGmThreads, 1) void gemm_kernel(GemmArgs a) {
    constexpr int BM = 16 * MB;
    constexpr int XPT = BM * kGroup / 8 / kGmThreads;  // 16-byte x loads per thread per group
    __shared__ __align__(16) uint16_t As[2][BM * kGmStride];

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

    // this wave's four row tiles (clamped to a valid tile; unused beyond N)
    int64_t tc[4];
    bool tok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t t = nt * 16 + wave * 4 + j;
        tok[j] = t < L.tiles;
        tc[j] = tok[j] ? t : L.tiles - 1;
    }

    uint4 xr[XPT];
    uint4 cw[4];
    float sc[4];
    auto load_group = [&](int64_t g) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int row = p * 16 + (tid >> 4), c = tid & 15;
            const int64_t gr = m0 + row < a.m ? m0 + row : a.m - 1;  // a valid row
            xr[p] = *reinterpret_cast<const uint4*>(a.x + gr * a.ldx + g * kGroup + c * 8);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            cw[j] = *reinterpret_cast<const uint4*>(a.packed + (tc[j] * L.groups + g) * kChunkBytes + lane * 16);
            sc[j] = scales[(tc[j] * L.groups + g) * kTileRows + r];
        }
    };
    // Rows past M hold a copy of the last row: they only feed accumulator
    // rows that are never stored.
    auto store_x = [&](int buf) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int row = p * 16 + (tid >> 4), c = tid & 15;
            *reinterpret_cast<uint4*>(&As[buf][row * kGmStride + c * 8]) = xr[p];
        }
    };

    f32x4_t acc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_group(g0);
    store_x(0);
    for (int gl = 0; gl < ng; ++gl) {
        const int buf = gl & 1;
        lds_barrier();  // As[buf] written; every wave is done with As[buf ^ 1]
        uint4 cur[4];
        float neg8s[4], s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            cur[j] = cw[j];
            s4[j] = tok[j] ? sc[j] : 0.0f;
            neg8s[j] = -8.0f * s4[j];
        }
        const bool more = gl + 1 < ng;
        if (more) load_group(g0 + gl + 1);
#pragma unroll
        for (int sk = 0; sk < 4; ++sk) {
            uint4 bop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = sk == 0 ? cur[j].x : sk == 1 ? cur[j].y : sk == 2 ? cur[j].z : cur[j].w;
                bop[j] = dequant_word<ACT>(w, s4[j], neg8s[j]);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const uint4 aop = *reinterpret_cast<const uint4*>(&As[buf][(i * 16 + r) * kGmStride + 32 * sk + 8 * kq]);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = gm_mfma<ACT>(aop, bop[j], acc[i][j]);
            }
        }
        if (more) store_x(buf ^ 1);
    }

    // --- epilogue: lane holds rows 4kq + e of column r of each 16 x 16 block
    const int64_t npad = a.ntiles * kGmBN;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t col = (nt * 16 + wave * 4 + j) * 16 + r;
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
    p.mtiles = ceil_div(m, kGmBM);
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
    if (act == kActBf16)
        gemm_kernel<kActBf16, kGmBM / 16><<<grid, block, 0, stream>>>(a);
    else
        gemm_kernel<kActF16, kGmBM / 16><<<grid, block, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(a.partials, p.splits, m, n, p.ntiles * kGmBN, a.bias, a.y, a.ldy, act, stream);
}

}  // namespace w4a16
