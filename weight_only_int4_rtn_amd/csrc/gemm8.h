// Eight-wave large-M kernel: a BM x BN output tile per workgroup (BM, BN in
// {128, 256}), eight waves of 64 lanes, one workgroup per CU.
//
// The K loop runs in stages of 64 (half a quantization group).  Per stage
// the workgroup stages in LDS the x tile (BM rows x 64, by direct
// global-to-LDS loads) and the B tile: the stage's weights dequantized to
// 16-bit MFMA operands, BN/16 tiles x 2 k-steps x 64 lanes x 16 bytes.  Each
// wave dequantizes BN/128 of the weight tiles (one word per lane per k-step,
// written where the reading lane finds it), so each weight is dequantized
// once per BM rows of x.  The waves form a WM x WN grid over the tile; a
// wave owns a (BM/WM) x (BN/WN) block of outputs as 16 x 16 MFMA blocks
// (v_mfma_f32_16x16x32_{bf16,f16}, FP32 accumulators):
//   256 x 256: 2 x 4 waves of 128 x 64     256 x 128: 4 x 2 waves of 64 x 64
//   128 x 256: 2 x 4 waves of  64 x 64     128 x 128: 2 x 4 waves of 64 x 32
// Each D = W . x^T block puts four consecutive outputs of one x row in a
// lane, which the epilogue stores together.
//
// Every stage runs its MFMA blocks, each followed by a slice of the next
// stage's dequantization (a finished word goes to the next B tile).  The
// barrier that publishes the next stage sits two blocks before the end of
// the stage: past it the x pieces of the stage three ahead are issued into
// the buffer just freed (three x buffers, so an x tile has two stages to
// arrive) and the next stage's first fragments are read, both overlapping
// the last two blocks (see `stage` below).  Measured on the 128 x 128 tile
// at M 1024, N 2560: with one stage of lead, x load latency set the stage
// time (the MFMA work of a stage is 512 clocks per SIMD there).
//
// INT8 weights: the same stages with a 16-byte run of each 1 KB chunk half
// per stage (byte codes, u = q + 128, fma(u, s, -128 s)).
//
// The epilogue adds the bias in FP32 and rounds once to the output dtype
// (through LDS as whole 16-byte rows when unsplit and aligned), or, for a K
// split, stores FP32 partial sums for the split-K reduce kernel.
//
// Stream-K (SK): the grid's workgroups take equal runs of the launch's
// tiles x 128-column groups, one segment per tile a run touches; the runs
// that share a tile add their FP32 sums through the workspace in K order
// (the fix-up at the end of the K loop below).
#pragma once

#include "gemm_common.h"

namespace w4a16 {

constexpr int kG8Threads = 512, kG8K = 64;

template <int BM, int BN>
struct G8Shape {
    static constexpr int WN = (BM == 256 && BN == 128) ? 2 : 4;  // waves along N
    static constexpr int WM = 8 / WN;                            // waves along M
    static constexpr int WTM = BM / WM, WTN = BN / WN;           // a wave's output block
    static constexpr int RB = WTM / 16, CB = WTN / 16;           // its 16 x 16 MFMA blocks
    static constexpr int NT = BN / 16;                           // 16-column weight tiles of the workgroup
    static constexpr int TPW = NT / 8;                           // weight tiles each wave dequantizes
    static constexpr int XP = BM / 64;                           // 1 KB x pieces each wave loads per stage
    static constexpr int SPI = 4 * TPW / RB;                     // dequantization quarter-words per MFMA block
    static constexpr int XSTAGE = BM * kG8K;                     // 16-bit elements of an x stage
    static constexpr int WSTAGE = NT * 2 * 64 * 16;              // bytes of a B stage
    static constexpr int RX = BM * 64 / BN;                      // output rows an x buffer holds (epilogue)
    static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile");
    static_assert(SPI * 2 * RB == 8 * TPW && SPI >= 1, "dequantization slices");
};

// x stage layout: row r holds its 64 columns as 8 segments of 16 bytes,
// segment c at position c ^ ((r >> 1) & 7): the 16 lanes of an operand read
// (16 consecutive rows, one segment) cover all 64 banks once.
__device__ inline int swz8(int row, int seg) { return row * kG8K + ((seg ^ ((row >> 1) & 7)) << 3); }

// Waits for all but N vector memory operations and for all LDS operations.
template <int N>
__device__ inline void wait_vm_lds() {
    static_assert(N >= 0 && N <= 15, "vmcnt range");
#define W4A16_WAIT(n) \
    if constexpr (N == n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)" ::: "memory");
    W4A16_WAIT(0) W4A16_WAIT(1) W4A16_WAIT(2) W4A16_WAIT(3) W4A16_WAIT(4) W4A16_WAIT(5) W4A16_WAIT(6)
    W4A16_WAIT(7) W4A16_WAIT(8) W4A16_WAIT(9) W4A16_WAIT(10) W4A16_WAIT(11) W4A16_WAIT(12) W4A16_WAIT(13)
    W4A16_WAIT(14) W4A16_WAIT(15)
#undef W4A16_WAIT
}

// One 16-byte LDS store of a B-tile word as a single vector store.  Through
// uint4 (a struct) the store is split into 4-byte pieces that the backend
// merges again, and the merged store of a tile's last word lost its alias
// information: the compiler then waited for every direct x load in flight
// before it.
__device__ inline void store_b16(uint8_t* p, uint4 v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4*>(p) = u32x4{v.x, v.y, v.z, v.w};
}

// BITS 8: INT8 chunks (two 1 KB halves, half h = stage 2g + h): a lane's
// k-step is two words of four byte codes, u = q + 128.
template <int ACT, bool STAGED, int BITS, int BM, int BN, bool SK>
__global__ __launch_bounds__(kG8Threads, 1) void gemm8_kernel(GemmArgs a) {
    using S = G8Shape<BM, BN>;
    // Arrays the lambdas below capture are sized by these fixed maxima, not
    // by the shape's constants: a captured array whose bound depends on the
    // template arguments makes the host pass drop the kernel's launch stub.
    constexpr int kMaxXP = 4, kMaxTPW = 2, kMaxRB = 8, kMaxCB = 4;
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    constexpr int RB = S::RB, CBL = S::CB, TPW = S::TPW, XP = S::XP, SPI = S::SPI, WTM = S::WTM, WN = S::WN,
                  NT = S::NT;
    // x buffers: three (an x tile issued two stages ahead), or two for INT8
    // at 256 x 256, whose register budget the third buffer's addresses
    // would overrun (spills)
    constexpr int XR = (BITS == 8 && BM == 256 && BN == 256) ? 2 : 3;
    __shared__ __align__(16) uint16_t X0[S::XSTAGE];
    __shared__ __align__(16) uint16_t X1[S::XSTAGE];
    __shared__ __align__(16) uint16_t X2[XR == 3 ? S::XSTAGE : 8];
    __shared__ __align__(16) uint8_t W0[S::WSTAGE];
    __shared__ __align__(16) uint8_t W1[S::WSTAGE];

    const Layout L(a.n, a.k, BITS);

    // One segment of work: groups g0 .. g0 + ng - 1 of output tile `tile`
    // (tile = mt + mtiles nt: consecutive tiles share weights), the K part
    // `split` of an equal split.
    auto segment = [&](const int64_t tile, const int split, const int64_t g0, const int ng) {
        const int64_t mt = tile % a.mtiles, nt = tile / a.mtiles;
        const int64_t m0 = mt * BM;
        const int nstages = 2 * ng;

        const int tid = threadIdx.x;
        const int wave = uniform(tid >> 6), lane = tid & 63;
        const int r = lane & 15, kq = lane >> 4;
        const int wm = wave / WN, wn = wave % WN;

        // x: rows m0 .. m0 + BM - 1 through a buffer resource ending at row M
        // (loads of rows past M fetch nothing; those rows only feed outputs never
        // stored).  Piece p of wave w fills stage rows 8 (XP w + p) .. +7; lane i
        // lands at row + i / 8, position i % 8.
        const int64_t rows_valid = min<int64_t>(BM, a.m - m0);
        const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(a.x + m0 * a.ldx, rows_valid * a.ldx * 2);
        static_assert(XP <= kMaxXP && TPW <= kMaxTPW && RB <= kMaxRB && CBL <= kMaxCB, "array maxima");
        uint32_t xoff[kMaxXP];
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int row = 8 * (XP * wave + p) + (lane >> 3);
            xoff[p] = uint32_t(row * a.ldx * 2 + (((lane & 7) ^ ((row >> 1) & 7)) << 4));
        }
        auto load_x = [&](uint16_t* dst, int s) {
            const int soff = uniform(int((g0 + (s >> 1)) * kGroup * 2 + (s & 1) * kG8K * 2));
#pragma unroll
            for (int p = 0; p < XP; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_ptr_t)(dst + (XP * wave + p) * 512), 16, xoff[p],
                                                         soff, 0, 0);
        };

        // Weights: this wave dequantizes the workgroup's tiles TPW w .. TPW w +
        // TPW - 1.  Tiles past N read the last tile again (clamped) with their
        // scales zeroed.
        const int64_t tw = nt * NT + TPW * wave;
        const int validw = int(min<int64_t>(TPW, max<int64_t>(0, L.tiles - tw)));
        const int64_t twfirst = min<int64_t>(tw, L.tiles - 1);
        const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(a.packed + twfirst * L.groups * CB, TPW * L.groups * CB);
        const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(
            a.packed + L.scale_offset() + twfirst * L.groups * kChunkScaleBytes, TPW * L.groups * kChunkScaleBytes);
        uint32_t woff[kMaxTPW], soff[kMaxTPW];
#pragma unroll
        for (int c = 0; c < TPW; ++c) {
            const int cc = c < validw ? c : (validw > 0 ? validw - 1 : 0);
            woff[c] = uint32_t(cc * L.groups * CB + lane * 16);
            soff[c] = uint32_t(cc * L.groups * kChunkScaleBytes + r * 4);
        }
        struct Words {
            uint32_t w[kMaxTPW][4 * H];  // INT8: half h in words 4h .. 4h + 3 (tiles c < TPW used)
            float s[kMaxTPW];
        };
        // one group's words and scales (groups past the split's end reload its
        // last group, keeping the count of loads in flight fixed)
        auto load_words = [&](Words& d, int gl) {
            const int64_t g = g0 + min(gl, ng - 1);
#pragma unroll
            for (int c = 0; c < TPW; ++c) {
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

        // FP32 accumulators of the wave's 16 x 16 blocks (i < RB, j < CBL used).
        // The MFMAs go through the compiler's builtin, so its hazard recognizer
        // pads only real hazards: the loop's operands come from LDS reads, and an
        // unconditional s_nop before each MFMA (inline assembly) cost 128 issue
        // slots per group.
        f32x4_t acc[kMaxRB][kMaxCB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CBL; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        Words wcur, wnext, wfut;
        // B-stage slot of (tile, k-step) for this lane
        auto wslot = [&](int tt, int ks) { return ((tt * 2 + ks) * 64 + lane) * 16; };

        // The first three x fragments and the k-step 0 weight fragments of a stage,
        // read as soon as the barrier that publishes the stage has passed (inside
        // the previous stage, overlapping its last MFMA blocks).
        uint4 xa[3], wa[kMaxCB];
        auto read_first = [&](const uint16_t* Xs, const uint8_t* Ws) {
#pragma unroll
            for (int f = 0; f < 3; ++f)
                xa[f] = *reinterpret_cast<const uint4*>(Xs + swz8(wm * WTM + (f % RB) * 16 + r, 4 * (f / RB) + kq));
#pragma unroll
            for (int j = 0; j < CBL; ++j) wa[j] = *reinterpret_cast<const uint4*>(Ws + wslot(wn * CBL + j, 0));
        };

        // One stage: F = 2 RB blocks of CBL MFMAs on fragments of the stage's
        // buffers (Xp, Wp), x fragments read three blocks ahead, the k-step 1
        // weight fragments RB / 2 + 1 blocks before they are needed.  Blocks 0 .. A - 1
        // (A = F - 2) also carry the dequantization slices of the next stage's
        // B tile into Wq.  After block A - 1 the wave has issued every read of
        // Xp / Wp and written its part of Wq: it waits for its own LDS traffic
        // and for the next stage's x pieces, and the workgroup barrier follows
        // there.  Past it nobody reads Xp any more, so the pieces of stage s + 3
        // go into Xp at once (with, at an even stage, the weight words two
        // groups ahead), and the next stage's first fragments are read while
        // blocks F - 2 and F - 1 run.  Fixed buffer roles per call let the
        // compiler tell the direct loads and B writes from the reads.  The last
        // stages load clamped copies into buffers nobody reads any more, which
        // keeps the loop free of branches.
        auto stage = [&](uint16_t* Xp, const uint8_t* Wp, uint16_t* Xq, uint8_t* Wq, int s, auto odd_c) {
            constexpr bool odd = decltype(odd_c)::value;
            constexpr int F = 2 * RB, A = F - 2, NS = 8 * TPW;
            // words of stage s + 1: the second half of this group, or the first
            // half of the next
            const Words& src = odd ? wnext : wcur;
            constexpr int h1 = odd ? 0 : 1;

            uint4 xf[4];
            xf[0] = xa[0];
            xf[1] = xa[1];
            xf[2] = xa[2];
            uint4 wf[kMaxCB], wg[kMaxCB];
#pragma unroll
            for (int j = 0; j < CBL; ++j) wf[j] = wa[j];
            auto read_x = [&](int f) {
                const int ks = f / RB, i = f % RB;
                return *reinterpret_cast<const uint4*>(Xp + swz8(wm * WTM + i * 16 + r, 4 * ks + kq));
            };
            uint32_t lo = 0, hi = 0;
            float c0 = 0.f, c4 = 0.f, c2 = 0.f, c6 = 0.f;
            uint4 out = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int ks = f / RB, i = f % RB;
                const uint4 xop = xf[f % 4];
                if (f + 3 < F) xf[(f + 3) % 4] = read_x(f + 3);
                if (f == RB / 2 - 1) {
#pragma unroll
                    for (int j = 0; j < CBL; ++j) wg[j] = *reinterpret_cast<const uint4*>(Wp + wslot(wn * CBL + j, 1));
                }
#pragma unroll
                for (int j = 0; j < CBL; ++j) acc[i][j] = gm_mfma<ACT>(ks == 0 ? wf[j] : wg[j], xop, acc[i][j]);
#pragma unroll
                for (int sl = f * NS / A; sl < (f + 1) * NS / A && f < A; ++sl) {
                    // quarter q of word (c, k-step kn) of stage s + 1
                    const int wi = sl >> 2;
                    const int c = wi >> 1, kn = wi & 1, q = sl & 3;
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
                            store_b16(Wq + wslot(TPW * wave + c, kn), out);
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
                            store_b16(Wq + wslot(TPW * wave + c, kn), out);
                        }
                    }
                }
                if (f == A - 1) {
                    // The next stage's x pieces were issued XR - 1 barriers ago.
                    // Since then (three buffers): at an even stage, the pieces of
                    // the stage after next (the previous, odd barrier); at an odd
                    // stage, the pieces of the stage after next and the words two
                    // groups ahead (the previous, even barrier).  Those may stay
                    // in flight; the words the next stage dequantizes (issued two
                    // barriers before an even stage) have landed with the rest.
                    // Two buffers: only the odd stage's words stay in flight.
                    if constexpr (odd)
                        wait_vm_lds<(XR - 2) * XP + TPW * (H + 1)>();
                    else
                        wait_vm_lds<(XR - 2) * XP>();
                    __builtin_amdgcn_s_barrier();
                    // keep the direct loads' M0 set-up below the barrier: hoisted
                    // above the last B write, it made the compiler wait there for
                    // every direct load in flight (x of the next stages)
                    __builtin_amdgcn_sched_barrier(0);
                    load_x(Xp, min(s + XR, nstages - 1));
                    if constexpr (!odd) load_words(wfut, (s >> 1) + 2);
                    read_first(Xq, Wq);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (odd) {
                wcur = wnext;
                wnext = wfut;
            }
        };

        // prologue: stage 0's x and the first two groups' words, stage 0's B
        // tile; then the x pieces of stages 1 and 2, the barrier that publishes
        // stage 0, and its first fragments (stage 0's barrier issues the words
        // two groups ahead)
        load_x(X0, 0);
        load_words(wcur, 0);
        load_words(wnext, 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < TPW; ++c) {
            const float sj = c < validw ? wcur.s[c] : 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                store_b16(W0 + wslot(TPW * wave + c, ks),
                          BITS == 8 ? dequant_word8<ACT>(wcur.w[c][2 * ks], wcur.w[c][2 * ks + 1], sj, -128.0f * sj)
                                        : dequant_word<ACT>(wcur.w[c][ks], sj, -8.0f * sj));
        }
        load_x(X1, min(1, nstages - 1));
        if constexpr (XR == 3) load_x(X2, min(2, nstages - 1));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        read_first(X0, W0);

        // B buffers and words alternate with the stage's parity (nstages is
        // even); with three x buffers, stage s reads X[s % 3]: six stages per
        // iteration, then the last two or four.  Each call names its buffers, so
        // the compiler can tell the direct loads into one x buffer from the
        // reads of another (through a pointer chosen at run time it would wait
        // for every direct load before the next read).
        if constexpr (XR == 3) {
            const int nfull = nstages - nstages % 6;
            for (int s = 0; s < nfull; s += 6) {
                stage(X0, W0, X1, W1, s, BoolC<false>{});
                stage(X1, W1, X2, W0, s + 1, BoolC<true>{});
                stage(X2, W0, X0, W1, s + 2, BoolC<false>{});
                stage(X0, W1, X1, W0, s + 3, BoolC<true>{});
                stage(X1, W0, X2, W1, s + 4, BoolC<false>{});
                stage(X2, W1, X0, W0, s + 5, BoolC<true>{});
            }
            if (nstages - nfull >= 2) {
                stage(X0, W0, X1, W1, nfull, BoolC<false>{});
                stage(X1, W1, X2, W0, nfull + 1, BoolC<true>{});
            }
            if (nstages - nfull >= 4) {
                stage(X2, W0, X0, W1, nfull + 2, BoolC<false>{});
                stage(X0, W1, X1, W0, nfull + 3, BoolC<true>{});
            }
        } else {
            for (int s = 0; s < nstages; s += 2) {
                stage(X0, W0, X1, W1, s, BoolC<false>{});
                stage(X1, W1, X0, W0, s + 1, BoolC<true>{});
            }
        }
        // the last stages' clamped x pieces land in LDS asynchronously: wait for
        // them before the epilogue reuses the buffers
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        if constexpr (SK) {
            // A stream-K segment over part of its tile's K: the runs that
            // touch the tile (wf .. wl, in K order) each store their FP32 sums
            // in a slot of the workspace, lane by lane as the registers hold
            // them, and count themselves in the tile's counter in the
            // workspace header.  The last to arrive adds the slots in K order
            // (the same order whichever run arrives last, so results repeat
            // bit for bit), zeroes the counter for the next call and runs the
            // epilogue; the others are done.  No workgroup waits for another.
            // The slots are written through and read past the L2s (device
            // scope: the 8 XCDs' L2s are not coherent with one another), so
            // the exchange needs no L2 write-back or invalidation, which
            // would evict the x tiles every other workgroup of the XCD is
            // reading.
            if (ng != L.groups) {
                const int64_t G = L.groups, UU = a.sk_units, P = gridDim.x, w = blockIdx.x;
                const int64_t ufirst = tile * G;
                const int64_t wf = ((ufirst + 1) * P - 1) / UU, wl = ((ufirst + G) * P - 1) / UU;
                // P slots when every run lies inside one tile, else 2 P
                const int64_t nslots = UU % P == 0 && G % (UU / P) == 0 ? P : 2 * P;
                const __amdgpu_buffer_rsrc_t slots = buffer_rsrc(a.partials, nslots * int64_t(BM * BN * 4));
                // byte offset of this lane's block (0, 0) in run v's slot for this tile: slot v, or
                // P + v when run v began in an earlier tile (only runs that cross a tile's end
                // use the upper half)
                auto slot = [&](int64_t v) -> uint32_t {
                    return uint32_t((v + (v * UU / P < ufirst ? P : 0)) * int64_t(BM * BN * 4)) +
                           uint32_t(wave * (RB * CBL * 1024) + lane * 16);
                };
                typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
                const uint32_t mine = slot(w);
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int j = 0; j < CBL; ++j)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), slots,
                                                               mine + (i * CBL + j) * 1024, 0, kCoherent);
                // the sums are at the device's coherence point before the count
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                int* const last = reinterpret_cast<int*>(X0);  // free: every wave is past its last stage
                if (tid == 0) {
                    const unsigned before =
                        __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    *last = before == unsigned(wl - wf);
                    if (*last) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                if (!*last) return;
                auto slot_sums = [&](uint32_t base, int b) {
                    return __builtin_bit_cast(f32x4_t,
                                              __builtin_amdgcn_raw_buffer_load_b128(slots, base + b * 1024, 0, kCoherent));
                };
                // blocks b = i CBL + j in batches of up to 16 (a batch of
                // another run's sums in flight at once; one batch on the
                // tiles offered, up to 256 x 128)
                constexpr int NB = RB * CBL, BATCH = NB < 16 ? NB : 16;
#pragma unroll
                for (int b0 = 0; b0 < NB; b0 += BATCH) {
                    if (w > wf) {
                        // runs before this one: (..(s_wf + s_wf+1) + ..) + own
                        f32x4_t pre[BATCH];
                        uint32_t base = slot(wf);
#pragma unroll
                        for (int b = 0; b < BATCH; ++b) pre[b] = slot_sums(base, b0 + b);
                        for (int64_t v = wf + 1; v < w; ++v) {
                            base = slot(v);
#pragma unroll
                            for (int b = 0; b < BATCH; ++b) pre[b] += slot_sums(base, b0 + b);
                        }
#pragma unroll
                        for (int b = 0; b < BATCH; ++b)
                            acc[(b0 + b) / CBL][(b0 + b) % CBL] = pre[b] + acc[(b0 + b) / CBL][(b0 + b) % CBL];
                    }
                    for (int64_t v = w + 1; v <= wl; ++v) {
                        const uint32_t base = slot(v);
#pragma unroll
                        for (int b = 0; b < BATCH; ++b)
                            acc[(b0 + b) / CBL][(b0 + b) % CBL] += slot_sums(base, b0 + b);
                    }
                }
            }
        }
        // --- epilogue: lane (r, kq) holds outputs 4kq .. 4kq + 3 of tile t0 + j
        // for x row r of row block i
        const int64_t npad = a.ntiles * BN;
        const int64_t t0 = nt * NT + wn * CBL;
        if constexpr (STAGED) {
            // Through LDS (one K split, 16-byte aligned rows): the BM x BN tile of
            // 16-bit outputs (2 BN bytes a row) fills the stage buffers (RX rows
            // in each x buffer, 64 in each B buffer) and leaves as whole rows in
            // 16-byte stores.  Within a row, 16-byte unit u sits at position
            // u ^ (row & (U - 1)), so the sixteen rows one write touches and the
            // units one row read touches spread over the banks.
            constexpr int RBY = 2 * BN, U = BN / 8, RX = S::RX;
            static_assert(2 * RX + 128 >= BM, "the output tile fits the stage buffers");
            __builtin_amdgcn_s_barrier();  // every wave is done with the last stage
            auto tile_row = [&](int row) -> uint8_t* {
                return row < RX            ? reinterpret_cast<uint8_t*>(X0) + row * RBY
                       : row < 2 * RX      ? reinterpret_cast<uint8_t*>(X1) + (row - RX) * RBY
                       : row < 2 * RX + 64 ? W0 + (row - 2 * RX) * RBY
                                           : W1 + (row - 2 * RX - 64) * RBY;
            };
            float ball[CBL][4];
            bias_tiles<ACT, CBL>(a.bias, t0, kq, a.n, ball);
#pragma unroll
            for (int j = 0; j < CBL; ++j) {
                const float* bv = ball[j];
                const int u = (wn * CBL + j) * 2 + (kq >> 1);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const int row = wm * WTM + i * 16 + r;
                    const f32x4_t v = acc[i][j];
                    *reinterpret_cast<uint2*>(tile_row(row) + ((u ^ (row & (U - 1))) << 4) + (kq & 1) * 8) =
                        make_uint2(pack2<ACT>(v[0] + bv[0], v[1] + bv[1]), pack2<ACT>(v[2] + bv[2], v[3] + bv[3]));
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            constexpr int RPI = kG8Threads / U;  // rows per pass
            const int u = tid % U;
            const int64_t col = nt * BN + u * 8;
#pragma unroll
            for (int it = 0; it < BM / RPI; ++it) {
                const int row = it * RPI + tid / U;
                const int64_t grow = m0 + row;
                const uint4 v = *reinterpret_cast<const uint4*>(tile_row(row) + ((u ^ (row & (U - 1))) << 4));
                if (grow >= a.m || col >= a.n) continue;
                uint16_t* dst = a.y + grow * a.ldy + col;
                if (col + 8 <= a.n) {
                    // streamed past the caches: a whole round of workgroups
                    // stores its tiles at once (measured 2-5 % faster)
                    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
                    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
                } else {
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                    for (int e = 0; e < 8 && col + e < a.n; ++e) dst[e] = uint16_t(w4[e >> 1] >> (16 * (e & 1)));
                }
            }
        } else {
            float ball[CBL][4];
            bias_tiles<ACT, CBL>(a.splits == 1 ? a.bias : nullptr, t0, kq, a.n, ball);
#pragma unroll
            for (int j = 0; j < CBL; ++j) {
                const int64_t c0 = (t0 + j) * 16 + 4 * kq;
                if (c0 >= a.n) continue;
                const bool full = c0 + 4 <= a.n;
                const float* bv = ball[j];
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const int64_t row = m0 + wm * WTM + i * 16 + r;
                    if (row >= a.m) continue;
                    const f32x4_t v = acc[i][j];
                    if (a.splits > 1) {
                        *reinterpret_cast<f32x4_t*>(a.partials + (int64_t(split) * a.m + row) * npad + c0) = v;
                    } else if (full && a.vec_store) {
                        *reinterpret_cast<uint2*>(a.y + row * a.ldy + c0) = make_uint2(
                            pack2<ACT>(v[0] + bv[0], v[1] + bv[1]), pack2<ACT>(v[2] + bv[2], v[3] + bv[3]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (c0 + e < a.n) a.y[row * a.ldy + c0 + e] = from_f32<ACT>(v[e] + bv[e]);
                    }
                }
            }
        }
    };

    if constexpr (!SK) {
        // one segment per workgroup: tile blockIdx / splits, K part blockIdx % splits
        const int split = int(blockIdx.x % unsigned(a.splits));
        const int64_t g0 = int64_t(split) * a.gps;
        segment(int64_t(blockIdx.x / unsigned(a.splits)), split, g0, int(min<int64_t>(a.gps, L.groups - g0)));
    } else {
        // Stream-K: the launch's tiles x groups units of work, taken tile by
        // tile in order, are cut into gridDim.x contiguous runs of equal
        // length (+-1); this workgroup computes run blockIdx.x, one segment
        // per tile the run touches.
        const int64_t G = L.groups, U = a.sk_units, P = gridDim.x, w = blockIdx.x;
        const int64_t uend = (w + 1) * U / P;
        for (int64_t u = w * U / P; u < uend;) {
            const int64_t tile = u / G, ga = u % G, gb = min<int64_t>(G, ga + (uend - u));
            if (u != w * U / P) __syncthreads();  // the previous segment's epilogue is done with LDS
            segment(tile, 0, ga, int(gb - ga));
            u += gb - ga;
        }
    }
}

// Launches the kernel variant of one tile (instantiated in the gemm8_*.hip
// file that defines that tile's launcher); sk: the stream-K variant.
template <int BM, int BN, bool SK>
static hipError_t launch_gemm8_sk(const GemmArgs& a, int bits, bool bf, bool staged, dim3 grid, hipStream_t stream) {
    const dim3 b8(kG8Threads);
#define W4A16_G8(ACT, ST, BITS) gemm8_kernel<ACT, ST, BITS, BM, BN, SK><<<grid, b8, 0, stream>>>(a)
    if (bits == 8) {
        if (staged) {
            if (bf) W4A16_G8(kActBf16, true, 8);
            else W4A16_G8(kActF16, true, 8);
        } else {
            if (bf) W4A16_G8(kActBf16, false, 8);
            else W4A16_G8(kActF16, false, 8);
        }
    } else {
        if (staged) {
            if (bf) W4A16_G8(kActBf16, true, 4);
            else W4A16_G8(kActF16, true, 4);
        } else {
            if (bf) W4A16_G8(kActBf16, false, 4);
            else W4A16_G8(kActF16, false, 4);
        }
    }
#undef W4A16_G8
    return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_gemm8(const GemmArgs& a, int bits, bool bf, bool staged, bool sk, dim3 grid,
                               hipStream_t stream) {
    // stream-K on 256 x 256 tiles: the run loop and the fix-up's second
    // set of sums take the K loop past its registers (spills); not offered
    if constexpr (BM * BN <= 256 * 128) {
        if (sk) return launch_gemm8_sk<BM, BN, true>(a, bits, bf, staged, grid, stream);
    } else {
        if (sk) return hipErrorInvalidValue;
    }
    return launch_gemm8_sk<BM, BN, false>(a, bits, bf, staged, grid, stream);
}

}  // namespace w4a16
