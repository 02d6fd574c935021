// Small-M forward on the matrix cores (M <= 16): the same weight stream as
// the v_dot2 kernel (gemv.hip), with the contraction done by MFMA.
//
// A workgroup of 4 or 8 waves owns one 16-row weight tile and a K split;
// wave w takes the split's groups w, w + waves, ...  Per chunk, a wave turns
// its four words into four B operands of v_mfma_f32_16x16x32_{bf16,f16} (the
// chunk layout is that operand layout: lane L holds column L % 16 of the
// tile, columns 8*(L/16) + j of each 32-wide k-step) and takes the matching
// A operands (row L % 16 of x, zero for rows >= M) from one of two places:
//  - staged (M <= 4 except on small layers of many row tiles, and M <= 8
//    with a fused activation): the workgroup stages its slice of x in LDS
//    once, activation applied there, one element per thread; the slice is
//    bounded (16 rows x 2048 columns), so larger M take more K splits;
//  - direct (otherwise): loaded straight from global memory with the chunk.
//    Each group of a split is used by one wave only, so there is nothing to
//    share: no staging barrier and no bound on the slice, hence fewer K
//    splits (M = 8, K = 16384, N = 2048: two splits instead of eight, 8.9
//    vs 9.7 us).  The loads cost four instructions per chunk however few rows are
//    live, and a fused activation runs in every lane of the 16 rows, which
//    is why small M keep the staged form (M = 4, same layer with SwiGLU:
//    19.7 vs 10.4 us).
// The packed pairs hold off + q exactly (off = 136 for bf16, 1032 for f16);
// four more MFMAs with the same A operands and a B operand of -off in every
// element (exact in both types) leave
//     sum_k x_k q_k
// in the accumulator, and the group's FP32 scale multiplies that into the
// FP32 totals.  (The extra MFMAs replace per-row sums of x and their
// cross-lane reductions: measured 2-25 % faster for M 3-16.)  The
// accumulator layout of the MFMA gives lane L the rows 4*(L/16) + i, i = 0..3,
// of column L % 16.  Per weight element this costs 7/8 of a VALU instruction
// for the nibble conversion, against 11/8 for the v_dot2 kernel at M = 1.
//
// Waves are summed through LDS in a fixed order.  K splits meet in a binary
// tree of exchange slots in the workspace header (as in gemv.hip), or, when
// the tree does not fit there, store FP32 partial sums for the split-K reduce
// kernel (reduce.hip).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

struct MgemvArgs {
    const uint16_t* x;
    int64_t ldx, m;
    const uint8_t* packed;
    int64_t n, k;
    const uint16_t* bias;
    uint16_t* y;
    int64_t ldy;
    unsigned long long* slots;  // [tiles][splits - 1][m * 16] exchange slots, zero before and after a call
    float* partials;            // [splits][m][tiles * 16] when the slots do not fit: split-K reduce kernel
    int splits, gps;
    int exchange;               // splits > 1: finish through the slots (else through partials)
};

constexpr int kMgChunks = 4;  // at most this many chunks per wave, all loaded up front
constexpr int kXRegs = 8;     // 16-byte x loads per thread while staging (4 waves)

template <int ACT>
__device__ inline f32x4_t mfma_16x16x32(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (ACT == kActBf16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// MMAX: rows of x staged (>= m, <= 16).  AF: activation fused into the x
// staging (ActFn; SwiGLU gate values sit k columns after the up values).
// BITS: 4 (INT4 chunks) or 8 (INT8 chunks, two 1 KB halves; each k-step's
// B operand is two words of byte codes, u = q + 128).
// WAVES: 4 or 8 waves per workgroup.
template <int MMAX, int ACT, int WAVES, int CPW, int AF, int BITS>
__global__ __launch_bounds__(64 * WAVES) void mgemv_kernel(MgemvArgs a) {
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    constexpr int kMgWaves = WAVES, kMgThreads = 64 * WAVES;
    // x staging: the slice is m <= 16 rows of at most 128 / m groups, i.e.
    // at most 2048 16-byte loads, kXRegs * 256 of them
    constexpr int XR = kXRegs * 4 / WAVES;
    extern __shared__ __align__(16) unsigned char smem[];
    const Layout L(a.n, a.k, BITS);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t t = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));
    const int klen = ng * kGroup;
    const int m = int(a.m);

    // x rows are padded by 16 bytes so the 16 rows an A-operand read touches
    // fall in different LDS banks.
    const int xstride = klen + 8;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                                      // [MMAX][xstride]
    float* red = reinterpret_cast<float*>(smem + size_t(MMAX) * (a.gps * kGroup + 8) * 2);   // [waves][16][16]

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;

    const uint8_t* cbase = a.packed + (t * L.groups + g0) * CB + lane * 16;
    const float* sbase = reinterpret_cast<const float*>(a.packed + L.scale_offset()) + (t * L.groups + g0) * kTileRows + r;

    // Every chunk of the wave (CPW of them) is loaded before any is used.
    // The loads are unconditional straight-line code (clamped addresses), so
    // the compiler's wait counts stay exact: each use waits for its own load.
    uint4 cw[CPW][H];
    float sc[CPW];

    // x slice first, then the first weight batch (loads complete in issue
    // order: staging waits for x only).  The plan keeps m * klen / 8 <=
    // kXRegs * threads.
    const int per_row = klen / 8;
    const int total = m * per_row;  // <= 2048: the plan keeps m * gps <= 128 groups
    const float inv_row = 1.0f / float(per_row);
    // zero-initialised so every register has a value on every path out of
    // the load loop: the compiler then keeps all x loads in flight together
    // (without it, it waited for each load before issuing the next)
    uint4 xv[XR];
#pragma unroll
    for (int j = 0; j < XR; ++j) xv[j] = make_uint4(0u, 0u, 0u, 0u);
    uint4 xgate[AF == kActFnSwiglu ? XR : 1];
#pragma unroll
    for (int j = 0; j < XR; ++j) {
        if (j * kMgThreads >= total) break;
        const int i = j * kMgThreads + tid;
        const int ic = i < total ? i : total - 1;
        const int row = div_small(ic, inv_row), c = ic - row * per_row;
        const uint16_t* src = a.x + row * a.ldx + g0 * kGroup + c * 8;
        xv[j] = *reinterpret_cast<const uint4*>(src);
        if constexpr (AF == kActFnSwiglu) xgate[j] = *reinterpret_cast<const uint4*>(src + a.k);
    }
    // keep the compiler from hoisting the weight loads above the x loads
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int gl = wave + u * kMgWaves;
        const int gc = gl < ng ? gl : ng - 1;  // a valid chunk; unused when gl >= ng
#pragma unroll
        for (int h = 0; h < H; ++h) cw[u][h] = *reinterpret_cast<const uint4*>(cbase + int64_t(gc) * CB + h * kChunkBytes);
        sc[u] = sbase[int64_t(gc) * kTileRows];
    }

    // Stage rows [0, m).
#pragma unroll
    for (int j = 0; j < XR; ++j) {
        if (j * kMgThreads >= total) break;
        const int i = j * kMgThreads + tid;
        const bool on = i < total;
        const int row = on ? div_small(i, inv_row) : 0, c = on ? i - row * per_row : 0;
        if constexpr (AF != kActFnNone) xv[j] = activate8<ACT, AF>(xv[j], xgate[AF == kActFnSwiglu ? j : 0]);
        if (on) *reinterpret_cast<uint4*>(xs + row * xstride + c * 8) = xv[j];
    }
    lds_barrier();

    constexpr float off = code_offset<ACT, BITS>();
    const uint32_t noff2 = uint32_t(from_f32<ACT>(-off)) * 0x00010001u;
    const uint4 bneg = make_uint4(noff2, noff2, noff2, noff2);  // -off in every element
    const bool row_on = r < m;
    const uint16_t* xrow = xs + (row_on ? r : 0) * xstride + 8 * kq;
    f32x4_t tot = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int gl = wave + u * kMgWaves;
        if (gl < ng) {
            uint32_t words[4 * H];
#pragma unroll
            for (int h = 0; h < H; ++h) {
                words[4 * h] = cw[u][h].x;
                words[4 * h + 1] = cw[u][h].y;
                words[4 * h + 2] = cw[u][h].z;
                words[4 * h + 3] = cw[u][h].w;
            }
            const float scale = sc[u];
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 av = make_uint4(0u, 0u, 0u, 0u);
                if (row_on) av = *reinterpret_cast<const uint4*>(xrow + gl * kGroup + 32 * s);
                const uint4 bv = bpairs<BITS, ACT>(words, s);
                acc = mfma_16x16x32<ACT>(av, bv, acc);
                acc = mfma_16x16x32<ACT>(av, bneg, acc);
            }
            tot[0] = fmaf(scale, acc[0], tot[0]);
            tot[1] = fmaf(scale, acc[1], tot[1]);
            tot[2] = fmaf(scale, acc[2], tot[2]);
            tot[3] = fmaf(scale, acc[3], tot[3]);
        }
    }

    // Lane holds rows 4kq + i of column r; sum the waves through LDS.
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * kq + i) * 16 + r] = tot[i];
    __syncthreads();
    const int orow = tid >> 4, ocol = tid & 15;  // the first 256 threads: 16 x 16 outputs
    if (orow >= m) return;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kMgWaves; ++w) v += red[(w * 16 + orow) * 16 + ocol];
    const int64_t col = t * kTileRows + ocol;
    if (a.splits > 1 && !a.exchange) {
        a.partials[(int64_t(split) * m + orow) * (L.tiles * kTileRows) + col] = v;
        return;
    }
    if (a.splits > 1) {
        // the split's parts meet in a binary tree of exchange slots, as in
        // the v_dot2 kernel (gemv.hip): one device atomic per level, the
        // second arrival adds (commutative, so reproducible) and climbs
        int node_base = 0, idx = split, width = a.splits;
        while (width > 1) {
            if (!((width & 1) && idx == width - 1)) {
                unsigned long long* slot =
                    a.slots + (t * (a.splits - 1) + node_base + (idx >> 1)) * (int64_t(m) * kTileRows) + tid;
                const unsigned long long mine = (1ull << 32) | __float_as_uint(v);
                const unsigned long long old =
                    __hip_atomic_exchange(slot, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((old >> 32) == 0ull) return;
                __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                v += __uint_as_float(uint32_t(old));
            }
            node_base += width >> 1;
            idx >>= 1;
            width = (width + 1) >> 1;
        }
    }
    if (col < a.n) {
        if (a.bias) v += to_f32<ACT>(a.bias[col]);
        a.y[orow * a.ldy + col] = from_f32<ACT>(v);
    }
}

// AF: activation fused into the A operands (ActFn; SwiGLU gate values sit k
// columns after the up values).  BITS: 4 (INT4 chunks) or 8 (INT8 chunks,
// two 1 KB halves; each k-step's B operand is two words of byte codes,
// u = q + 128).  WAVES: 4 or 8 waves per workgroup; CPW: chunks per wave.
template <int ACT, int WAVES, int CPW, int AF, int BITS>
__global__ __launch_bounds__(64 * WAVES) void mgemv_direct_kernel(MgemvArgs a) {
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    constexpr bool GATE = AF == kActFnSwiglu;
    extern __shared__ __align__(16) unsigned char smem[];
    const Layout L(a.n, a.k, BITS);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t t = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));
    const int m = int(a.m);
    float* red = reinterpret_cast<float*>(smem);  // [waves][16][16]

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const bool row_on = r < m;

    const uint8_t* cbase = a.packed + (t * L.groups + g0) * CB + lane * 16;
    const float* sbase = reinterpret_cast<const float*>(a.packed + L.scale_offset()) + (t * L.groups + g0) * kTileRows + r;
    const uint16_t* xrow = a.x + int64_t(row_on ? r : 0) * a.ldx + g0 * kGroup + 8 * kq;

    // A wave issues its first PF chunks (codes, scale and the A operands of
    // x) up front and each further chunk while computing the chunk PF before
    // it: a wave stalls at issue once the memory pipeline is full, so with
    // every chunk issued at once it would compute nothing until its stream
    // had almost arrived.  The chunk loads are unconditional straight-line
    // code (clamped addresses) and the x loads are masked to the lanes of
    // rows < M, which every wave has, so each use waits for its own load.  A
    // SwiGLU chunk holds twice the x registers: a window of 2 keeps the wave
    // within 128 VGPRs.
    constexpr int PF = CPW < (GATE ? 2 : 4) ? CPW : (GATE ? 2 : 4);
    uint4 cw[CPW][H];
    float sc[CPW];
    uint4 xa[CPW][4];
    uint4 xg[GATE ? CPW : 1][4];
    auto load_chunk = [&](int u) {
        const int gl = wave + u * WAVES;
        const int gc = gl < ng ? gl : ng - 1;  // a valid chunk; unused when gl >= ng
#pragma unroll
        for (int h = 0; h < H; ++h) cw[u][h] = load_stream16(cbase + int64_t(gc) * CB + h * kChunkBytes);
        sc[u] = sbase[int64_t(gc) * kTileRows];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            xa[u][s] = make_uint4(0u, 0u, 0u, 0u);
            if constexpr (GATE) xg[u][s] = make_uint4(0u, 0u, 0u, 0u);
            if (row_on) {
                const uint16_t* src = xrow + gc * kGroup + 32 * s;
                xa[u][s] = *reinterpret_cast<const uint4*>(src);
                if constexpr (GATE) xg[u][s] = *reinterpret_cast<const uint4*>(src + a.k);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) load_chunk(u);

    constexpr float off = code_offset<ACT, BITS>();
    const uint32_t noff2 = uint32_t(from_f32<ACT>(-off)) * 0x00010001u;
    const uint4 bneg = make_uint4(noff2, noff2, noff2, noff2);  // -off in every element
    f32x4_t tot = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int gl = wave + u * WAVES;
        if (u + PF < CPW) load_chunk(u + PF);
        if (gl < ng) {
            uint32_t words[4 * H];
#pragma unroll
            for (int h = 0; h < H; ++h) {
                words[4 * h] = cw[u][h].x;
                words[4 * h + 1] = cw[u][h].y;
                words[4 * h + 2] = cw[u][h].z;
                words[4 * h + 3] = cw[u][h].w;
            }
            const float scale = sc[u];
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 av = xa[u][s];
                if constexpr (AF != kActFnNone) av = activate8<ACT, AF>(av, xg[GATE ? u : 0][s]);
                const uint4 bv = bpairs<BITS, ACT>(words, s);
                acc = mfma_16x16x32<ACT>(av, bv, acc);
                acc = mfma_16x16x32<ACT>(av, bneg, acc);
            }
            tot[0] = fmaf(scale, acc[0], tot[0]);
            tot[1] = fmaf(scale, acc[1], tot[1]);
            tot[2] = fmaf(scale, acc[2], tot[2]);
            tot[3] = fmaf(scale, acc[3], tot[3]);
        }
    }

    // Lane holds rows 4kq + i of column r; sum the waves through LDS.
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * kq + i) * 16 + r] = tot[i];
    __syncthreads();
    const int orow = tid >> 4, ocol = tid & 15;  // the first 256 threads: 16 x 16 outputs
    if (orow >= m) return;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[(w * 16 + orow) * 16 + ocol];
    const int64_t col = t * kTileRows + ocol;
    if (a.splits > 1 && !a.exchange) {
        a.partials[(int64_t(split) * m + orow) * (L.tiles * kTileRows) + col] = v;
        return;
    }
    if (a.splits > 1) {
        // the split's parts meet in a binary tree of exchange slots, as in
        // the v_dot2 kernel (gemv.hip): one device atomic per level, the
        // second arrival adds (commutative, so reproducible) and climbs
        int node_base = 0, idx = split, width = a.splits;
        while (width > 1) {
            if (!((width & 1) && idx == width - 1)) {
                unsigned long long* slot =
                    a.slots + (t * (a.splits - 1) + node_base + (idx >> 1)) * (int64_t(m) * kTileRows) + tid;
                const unsigned long long mine = (1ull << 32) | __float_as_uint(v);
                const unsigned long long old =
                    __hip_atomic_exchange(slot, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((old >> 32) == 0ull) return;
                __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                v += __uint_as_float(uint32_t(old));
            }
            node_base += width >> 1;
            idx >>= 1;
            width = (width + 1) >> 1;
        }
    }
    if (col < a.n) {
        if (a.bias) v += to_f32<ACT>(a.bias[col]);
        a.y[orow * a.ldy + col] = from_f32<ACT>(v);
    }
}

// Staged plans: split K only when the row tiles cannot fill the chip; the x
// slice stays within 16 rows x 2048 columns; at most 4 chunks per wave (a
// split of more than 16 INT4 groups takes 8 waves: measured faster than 4
// waves of 8 chunks, as for the v_dot2 kernel).
//
// Direct plans: splits of up to 64 INT4 groups (8 waves of up to 8 chunks,
// issued a window ahead) or 16 INT8 groups (4 waves of up to 4 chunks of
// twice the registers), balanced; a split of at most 16 INT4 groups runs on
// 4 waves.  K is split only as far as a split's registers require: a split
// merely to fill the chip adds an exchange level (M = 16, K = 2048, N = 2560:
// 5.2 us unsplit, 5.35 in two).
MgemvPlan plan_mgemv(int64_t m, int64_t n, int64_t k, int bits, int act_fn) {
    MgemvPlan p{};
    const Layout L(n, k, bits);
    // small layers of >= 128 row tiles take the direct form from M = 1 (M = 3
    // and 4, K = 2048, N = 2560: 4.3 and 4.4 us against 4.6 staged); with
    // fewer tiles the staged plan's K split fills more of the chip (M = 4,
    // K = 4096, N = 1024: 4.8 against 5.0 direct)
    const bool small = n * k <= (int64_t(8) << 20) && L.tiles >= 128;
    p.direct = (act_fn == kActFnNone && (m > 4 || small)) || m > 8;
    if (p.direct) {
        const int64_t cap = bits == 8 ? 16 : 64;
        int64_t splits = ceil_div(L.groups, cap);
        // fewer than 128 row tiles: split K towards 256 workgroups, down to
        // 8 groups per split (M = 16, K = 4096, N = 1024: 5.3 us in four
        // splits, 6.7 unsplit on 64 workgroups)
        if (L.tiles < 128) {
            const int64_t want = ceil_div(int64_t(256), L.tiles), most = L.groups / 8;
            const int64_t more = want < most ? want : most;
            if (more > splits) splits = more;
        }
        const int64_t gps = ceil_div(L.groups, splits);
        p.mmax = 16;
        p.gps = int(gps);
        p.waves = (bits == 4 && gps > 16) ? 8 : 4;
        const int64_t per_wave = ceil_div(gps, p.waves);
        p.cpw = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : 8;
        p.lds = size_t(p.waves) * 256 * 4;
    } else {
        p.mmax = m <= 4 ? 4 : 8;
        int64_t splits = 1;
        if (L.tiles < 512) splits = ceil_div(512, L.tiles);
        int64_t gps = ceil_div(L.groups, splits);
        if (gps < 8) gps = 8;
        int64_t max_gps = 128 / m;  // x slice <= 2048 16-byte loads
        // chunks per workgroup held in registers (INT8 chunks take twice the registers)
        const int64_t wg_chunks = bits == 8 ? kMgChunks * 4 : kMgChunks * 8;
        if (max_gps > wg_chunks) max_gps = wg_chunks;
        if (gps > max_gps) gps = max_gps;
        if (gps > L.groups) gps = L.groups;
        p.gps = int(gps);
        p.waves = gps > 4 * kMgChunks ? 8 : 4;
        const int64_t per_wave = ceil_div(gps, p.waves);
        p.cpw = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : 4;
        p.lds = size_t(p.mmax) * (gps * kGroup + 8) * 2 + size_t(p.waves) * 256 * 4;
    }
    p.splits = int(ceil_div(L.groups, int64_t(p.gps)));
    const int64_t slots = L.tiles * (p.splits - 1) * m * kTileRows;
    p.exchange = p.splits > 1 && slots * 8 <= int64_t(kSyncBytes);
    p.workspace = p.splits == 1 ? 0
                  : p.exchange ? kSyncBytes
                               : kSyncBytes + size_t(p.splits) * m * L.tiles * kTileRows * 4;
    return p;
}

PlanInfo describe_mgemv(int64_t m, int64_t n, int64_t k, int bits, int act_fn) {
    const MgemvPlan p = plan_mgemv(m, n, k, bits, act_fn);
    const Layout L(n, k, bits);
    return {p.waves, int(m), kTileRows, p.splits, p.gps, L.tiles * p.splits, p.splits > 1 && !p.exchange};
}

template <int ACT, int AF, int BITS>
static void launch_direct(const MgemvArgs& a, const MgemvPlan& p, dim3 grid, dim3 block, hipStream_t stream) {
    if (p.waves == 8) {
        // 17..64 INT4 groups per split (the plan gives INT8 4 waves)
        if constexpr (BITS == 4) {
            if (p.cpw == 8) mgemv_direct_kernel<ACT, 8, 8, AF, BITS><<<grid, block, p.lds, stream>>>(a);
            else mgemv_direct_kernel<ACT, 8, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a);
        }
        return;
    }
    switch (p.cpw) {
        case 1: mgemv_direct_kernel<ACT, 4, 1, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
        case 2: mgemv_direct_kernel<ACT, 4, 2, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
        default: mgemv_direct_kernel<ACT, 4, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
    }
}

template <int MMAX, int ACT, int AF, int BITS>
static void launch_staged(const MgemvArgs& a, const MgemvPlan& p, dim3 grid, dim3 block, hipStream_t stream) {
    if (p.waves == 8) {
        // 17..32 groups per split (INT4 only): 8 waves of 4 chunks
        if constexpr (BITS == 4) mgemv_kernel<MMAX, ACT, 8, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a);
        return;
    }
    switch (p.cpw) {
        case 1: mgemv_kernel<MMAX, ACT, 4, 1, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
        case 2: mgemv_kernel<MMAX, ACT, 4, 2, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
        default: mgemv_kernel<MMAX, ACT, 4, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
    }
}

template <int ACT, int AF, int BITS>
static hipError_t launch_one(const MgemvArgs& a, const MgemvPlan& p, hipStream_t stream) {
    const Layout L(a.n, a.k, BITS);
    if (BITS == 8 && p.waves == 8) return hipErrorInvalidValue;
    const dim3 grid(unsigned(L.tiles * p.splits)), block(unsigned(64 * p.waves));
    if (p.direct) launch_direct<ACT, AF, BITS>(a, p, grid, block, stream);
    else if (p.mmax == 4) launch_staged<4, ACT, AF, BITS>(a, p, grid, block, stream);
    else launch_staged<8, ACT, AF, BITS>(a, p, grid, block, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1 || p.exchange) return e;
    return launch_splitk_reduce(a.partials, p.splits, a.m, a.n, L.tiles * kTileRows, a.bias, a.y, a.ldy,
                                ACT, stream);
}

template <int ACT, int BITS>
static hipError_t launch_af(const MgemvArgs& a, const MgemvPlan& p, int act_fn, hipStream_t stream) {
    switch (act_fn) {
        case kActFnSwiglu: return launch_one<ACT, kActFnSwiglu, BITS>(a, p, stream);
        case kActFnGeluTanh: return launch_one<ACT, kActFnGeluTanh, BITS>(a, p, stream);
        default: return launch_one<ACT, kActFnNone, BITS>(a, p, stream);
    }
}

template <int BITS>
static hipError_t launch_bits(const MgemvArgs& a, const MgemvPlan& p, int act, int act_fn, hipStream_t stream) {
    return act == kActBf16 ? launch_af<kActBf16, BITS>(a, p, act_fn, stream)
                           : launch_af<kActF16, BITS>(a, p, act_fn, stream);
}

hipError_t launch_mgemv(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                        const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                        hipStream_t stream) {
    const MgemvPlan p = plan_mgemv(m, n, k, bits, act_fn);
    MgemvArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.m = m;
    a.packed = static_cast<const uint8_t*>(packed);
    a.n = n;
    a.k = k;
    a.bias = static_cast<const uint16_t*>(bias);
    a.y = static_cast<uint16_t*>(y);
    a.ldy = ldy;
    a.slots = static_cast<unsigned long long*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSyncBytes);
    a.splits = p.splits;
    a.gps = p.gps;
    a.exchange = p.exchange;
    return bits == 8 ? launch_bits<8>(a, p, act, act_fn, stream) : launch_bits<4>(a, p, act, act_fn, stream);
}

}  // namespace w4a16
