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
// Two kernel families; the planner below picks one, its tile and its K split
// per shape:
//   gemm_kernel<ACT, MB> (this file): 16 MB x 256 tiles (MB = 4: 64 rows),
//     four waves (two workgroups per CU); wave w owns 64 columns and all the
//     rows, and dequantizes its own chunks in registers between its MFMAs.
//     (A 128-row variant measured slower than the eight-wave tiles on every
//     large-M shape once those stage x three deep, and was dropped.)
//   gemm8_kernel (gemm8.h): 256 x 256, 256 x 128, 128 x 256 or 128 x 128
//     tiles, eight waves; the workgroup dequantizes each weight once into an
//     LDS operand tile that all waves read.
// Both stage x in LDS by direct-to-LDS buffer loads (rows past M fall
// outside the buffer and fetch nothing), double-buffered with one barrier
// per stage, and spread the next stage's loads and dequantization between
// the MFMAs of the current one.  The MFMAs go through the compiler builtin,
// which pads only the hazards that are there.
//
// INT8 weights (W8A16) run on gemm8_kernel only: the same stages with a
// 16-byte run of each 1 KB chunk half per stage (byte codes, u = q + 128,
// fma(u, s, -128 s)).
//
// The epilogue adds the bias in FP32 and rounds once to the output dtype, or,
// for a K split, stores FP32 partial sums for the split-K reduce kernel.
//
// Stream-K (the explicit W4A16_PATH_GEMM_STREAMK path): gemm8_kernel on up
// to 256 x 128 tiles with the launch's tiles x groups cut into one run of
// equal length per CU; runs that share a tile add their sums in-kernel
// (see gemm8.h).  The planner itself keeps to the equal splits, which
// measured faster (plan_gemm below).
#include <algorithm>

#include "gemm_common.h"

namespace w4a16 {

constexpr int kGmBN = 256, kGmThreads = 256;  // rows per workgroup: 16 * MB
#ifndef GM_PREFETCH
#define GM_PREFETCH 2
#endif
constexpr int kGmPrefetch = GM_PREFETCH;  // A fragments read ahead of their MFMAs

// LDS layout of an x tile: row r of BM rows holds its 128 columns as 16
// segments of 16 bytes, segment c stored at position c ^ (r & 15).  The 16
// lanes of an A-operand read (rows r0..r0+15, one segment each) then touch 16
// different bank groups, with no padding, so each 1 KB piece of the tile can
// be filled by one global_load_lds_dwordx4 (lane i -> LDS bytes 16i..16i+15).
__device__ inline int swz(int row, int seg) { return row * 128 + ((seg ^ (row & 15)) << 3); }

// A wave's four 1 KB weight chunks of one group and their dequantization
// into MFMA B operands, one k-step (one word per lane per chunk) at a time.
template <int ACT>
struct GroupWords {
    uint4 w[4];      // this lane's 16 bytes of each chunk: word s = k-step s
    float s[4], o[4];  // scale and -8 * scale per chunk
};

template <int ACT, int MB>
__global__ __launch_bounds__(kGmThreads, 2) void gemm_kernel(GemmArgs a) {
    static_assert(MB == 4, "64-row tiles");
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
                for (int j = 0; j < 4; ++j) acc[i][j] = gm_mfma<ACT>(bc[j], aop, acc[i][j]);
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

    // --- epilogue.  Each 16 x 16 block is D = W . x^T: lane (r, kq) holds
    // outputs 4kq .. 4kq + 3 of tile t0 + j for x row r of row block i, four
    // consecutive columns (one 8-byte store, 16 bytes for FP32 partials).
    const int64_t npad = a.ntiles * kGmBN;
    float ball[4][4];
    bias_tiles<ACT, 4>(a.splits == 1 ? a.bias : nullptr, t0, kq, a.n, ball);
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

// --- planning -----------------------------------------------------------
//
// The plan is a pure function of (m, n, k, bits): no autotuning and no
// runtime state, so the workspace size is fixed by the shape.  Candidates:
// the eight-wave kernel with 256 x 256, 256 x 128, 128 x 256 or 128 x 128
// tiles and the four-wave kernel with 64 x 256 tiles (two
// workgroups per CU), each with every K split into equal parts.  A
// candidate's time is modelled as
//     rounds x (tile work / (w x per-CU peak) + fixed)  [+ partials / bw + reduce]
// rounds: the waves of workgroups the CUs run; tile work: 2 bm bn (K / split);
// fixed: a round's first loads and epilogue; for a split, the FP32 partial
// sums written and read back by the reduce kernel plus its launch.  The
// weights w and the three constants were fitted to the measured times of
// every tiling and split on 14 large-M shapes (MI355X, launches over >= 1 GiB
// of distinct weights); with them the model picks the fastest measured
// candidate on all 14.  Measured examples (us): 1024 x 2560 x 2048 fp16,
// 128 x 128 tiles unsplit 22.7 (256 x 128 in three: 30.3); 1024 x 2048 x
// 16384, 256 x 128 tiles split in four 76.6 (256 x 256 in eight: 84.5);
// 4096 x 2048 x 16384, 256 x 256 in two 233.7 (unsplit: 237.3).
namespace {

struct GemmTile {
    int waves, bm, bn;
    double w;    // fitted weight: the fraction of a CU's MFMA peak a workgroup's work runs at
    int per_cu;  // workgroups one CU runs at once
};

constexpr GemmTile kTiles[] = {
    {8, 256, 256, 0.70, 1}, {8, 256, 128, 0.499, 1}, {8, 128, 256, 0.428, 1},
    {8, 128, 128, 0.289, 1}, {4, 64, 256, 0.381, 2},
};
constexpr double kRoundFixed = 4.0e-6;     // s per round of workgroups
constexpr double kPartialBw = 3.93e12;     // B/s for partial sums written + read back
constexpr double kReduceLaunch = 3.48e-6;  // s

double tile_cost(const GemmTile& t, int64_t m, int64_t n, int64_t groups, int64_t splits, int64_t* gps_out,
                 int64_t* splits_out) {
    const int64_t tiles = ceil_div(m, t.bm) * ceil_div(n, t.bn);
    const int64_t gps = ceil_div(groups, splits);
    const int64_t parts = ceil_div(groups, gps);
    const int64_t wgs = tiles * parts;
    const int64_t rounds = ceil_div(wgs, int64_t(256) * t.per_cu);
    const double cu_peak = 2.5e15 / 256.0;
    const double t_wg = 2.0 * t.bm * t.bn * double(gps * kGroup) / (t.w * cu_peak / t.per_cu);
    double cost = double(rounds) * (t_wg + kRoundFixed);
    if (parts > 1) cost += 2.0 * double(parts) * double(m) * double(n) * 4.0 / kPartialBw + kReduceLaunch;
    *gps_out = gps;
    *splits_out = parts;
    return cost;
}

}  // namespace

// A stream-K plan of bm x bn tiles (eight waves): the tiles x groups units
// cut into `runs` runs of equal length (+-1), one workgroup each.
// Workspace: the header (one counter per tile) and an FP32 tile slot per
// run, two when runs cross tile ends.  256 x 256 tiles are not offered (see
// launch_gemm8).
constexpr int64_t kSkMaxRuns = 256;  // one run per CU

GemmPlan plan_gemm_sk(int64_t m, int64_t n, int64_t k, int bits, int bm, int bn, int64_t runs) {
    GemmPlan p{};
    const Layout L(n, k, bits);
    p.waves = 8;
    p.bm = bm;
    p.bn = bn;
    p.mb = bm / 16;
    p.mtiles = ceil_div(m, bm);
    p.ntiles = ceil_div(n, bn);
    p.splits = 1;
    p.sk = true;
    const int64_t units = p.mtiles * p.ntiles * L.groups;
    p.wgs = std::min(runs, units);
    p.gps = int(ceil_div(units, p.wgs));
    // runs that each lie inside one tile: units / runs whole and a divisor of the tile's groups
    const bool inside = units % p.wgs == 0 && L.groups % (units / p.wgs) == 0;
    p.workspace = kSyncBytes + size_t((inside ? 1 : 2) * p.wgs) * bm * bn * 4;
    return p;
}

namespace {

// The tile counters live in the workspace header.
bool sk_fits(int64_t m, int64_t n, int bm, int bn) {
    return ceil_div(m, bm) * ceil_div(n, bn) <= int64_t(kSyncBytes / 4);
}

GemmPlan plan_gemm_dp(int64_t m, int64_t n, int64_t k, int bits) {
    GemmPlan p{};
    const Layout L(n, k, bits);
    double best = 1e30;
    for (const GemmTile& t : kTiles) {
        if (bits == 8 && t.waves != 8) continue;  // INT8 weights: the eight-wave kernel only
        for (int64_t s = 1; s <= L.groups && s <= 32; ++s) {
            int64_t gps = 0, parts = 0;
            const double c = tile_cost(t, m, n, L.groups, s, &gps, &parts);
            if (parts != s) continue;  // the same split as a smaller s
            if (c < best * (1.0 - 1e-9)) {
                best = c;
                p.waves = t.waves;
                p.bm = t.bm;
                p.bn = t.bn;
                p.gps = int(gps);
                p.splits = int(parts);
            }
        }
    }
    p.mb = p.bm / 16;
    p.mtiles = ceil_div(m, p.bm);
    p.ntiles = ceil_div(n, p.bn);
    p.sk = false;
    p.wgs = p.mtiles * p.ntiles * p.splits;
    p.workspace = p.splits > 1 ? kSyncBytes + size_t(p.splits) * m * p.ntiles * p.bn * 4 : 0;
    return p;
}

}  // namespace

// The forced stream-K path: the equal-split planner's tile where the
// stream-K kernel takes it (256 x 256 -> 256 x 128, the four-wave 64 x 256
// -> 128 x 256), one run per CU.
GemmPlan plan_gemm_streamk(int64_t m, int64_t n, int64_t k, int bits) {
    const GemmPlan d = plan_gemm_dp(m, n, k, bits);
    const int bm = d.waves == 4 ? 128 : d.bm, bn = d.waves == 4 ? 256 : (d.bm == 256 ? 128 : d.bn);
    return plan_gemm_sk(m, n, k, bits, bm, bn, kSkMaxRuns);
}

// The planner's choice: the equal-split candidates above.  Stream-K is not
// among them: measured on MI355X it was slower than the equal split with
// the reduce kernel on every shape tried.  A run's second segment restarts
// the stage pipeline, and the fix-up puts the slot round trips of the last
// run to finish each tile on the launch's tail, on the few workgroups that
// finish tiles, where the reduce kernel spreads that pass over every CU
// (1024 x 2560 x 2048: 23.7 us unsplit on 128 x 128 tiles, 28.1 us as
// stream-K; 1024 x 16384 x 2048 on 256 x 128 tiles in four parts: 77 us
// with the reduce kernel, 80 us with the parts added in-kernel).
GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k, int bits) { return plan_gemm_dp(m, n, k, bits); }

PlanInfo describe_gemm(int64_t m, int64_t n, int64_t k, int bits, bool streamk) {
    const GemmPlan p = streamk ? plan_gemm_streamk(m, n, k, bits) : plan_gemm(m, n, k, bits);
    if (!p.sk) return {p.waves, p.bm, p.bn, p.splits, p.gps, p.wgs, p.splits > 1, false};
    // the most runs that share one tile
    const int64_t G = Layout(n, k, bits).groups, U = p.mtiles * p.ntiles * G, P = p.wgs;
    int64_t most = 1;
    for (int64_t w = 0; w < P; ++w) {
        const int64_t u0 = w * U / P;
        if (u0 % G == 0) continue;  // only a run that begins inside a tile shares it with earlier runs
        const int64_t t = u0 / G;
        most = std::max(most, ((t * G + G) * P - 1) / U - ((t * G + 1) * P - 1) / U + 1);
    }
    return {p.waves, p.bm, p.bn, int(most), p.gps, p.wgs, false, true};
}

hipError_t launch_gemm(const void* x, int act, int bits, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace, bool streamk,
                       hipStream_t stream) {
    const GemmPlan p = streamk ? plan_gemm_streamk(m, n, k, bits) : plan_gemm(m, n, k, bits);
    // the x tile's buffer resource takes 32-bit byte offsets
    if (int64_t(p.bm) * ldx * 2 > int64_t(0xFFFFFFFF)) return hipErrorInvalidValue;
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
    a.counters = static_cast<unsigned*>(workspace);
    a.sk_units = p.sk ? p.mtiles * p.ntiles * (k / kGroup) : 0;
    const dim3 grid(unsigned(p.wgs)), block(kGmThreads);
    const bool bf = act == kActBf16;
    if (p.waves == 8) {
        const bool staged = p.splits == 1 && a.vec16;
        hipError_t e;
        if (p.bm == 256 && p.bn == 256) e = launch_gemm8_256x256(a, bits, bf, staged, p.sk, grid, stream);
        else if (p.bm == 256) e = launch_gemm8_256x128(a, bits, bf, staged, p.sk, grid, stream);
        else if (p.bn == 256) e = launch_gemm8_128x256(a, bits, bf, staged, p.sk, grid, stream);
        else e = launch_gemm8_128x128(a, bits, bf, staged, p.sk, grid, stream);
        if (e != hipSuccess) return e;
    } else {
        if (bf) gemm_kernel<kActBf16, 4><<<grid, block, 0, stream>>>(a);
        else gemm_kernel<kActF16, 4><<<grid, block, 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(a.partials, p.splits, m, n, p.ntiles * p.bn, a.bias, a.y, a.ldy, act, stream);
}

}  // namespace w4a16
