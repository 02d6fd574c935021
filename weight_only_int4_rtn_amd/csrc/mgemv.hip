// Small-M forward on the matrix cores (M <= 16): the same weight stream as
// the v_dot2 kernel (gemv.hip), with the contraction done by MFMA.
//
// A workgroup of 4 or 8 waves owns one 16-row weight tile and a K split.  The
// workgroup stages its slice of x (M rows) in LDS once.  Per chunk, a wave
// turns its four words into
// four B operands of v_mfma_f32_16x16x32_{bf16,f16} (the chunk layout is that
// operand layout: lane L holds column L % 16 of the tile, columns
// 8*(L/16) + j of each 32-wide k-step), reads the matching A operands (row
// L % 16 of x, zero for rows >= M) from LDS, and runs four MFMAs into a fresh
// accumulator.  The packed pairs hold off + q exactly (off = 136 for bf16,
// 1032 for f16); four more MFMAs with the same A operands and a B operand of
// -off in every element (exact in both types) leave
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

// Same plan shape as the v_dot2 kernel: split K only when the row tiles
// cannot fill the chip; the x slice stays within 16 rows x 2048 columns; at
// most 4 chunks per wave (a split of more than 16 INT4 groups takes 8 waves:
// measured faster than 4 waves of 8 chunks, as for the v_dot2 kernel).
MgemvPlan plan_mgemv(int64_t m, int64_t n, int64_t k, int bits) {
    MgemvPlan p{};
    const Layout L(n, k, bits);
    p.mmax = m <= 4 ? 4 : m <= 8 ? 8 : 16;
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
    p.splits = int(ceil_div(L.groups, gps));
    p.waves = gps > 4 * kMgChunks ? 8 : 4;
    const int64_t per_wave = ceil_div(gps, p.waves);
    p.cpw = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : 4;
    p.lds = size_t(p.mmax) * (gps * kGroup + 8) * 2 + size_t(p.waves) * 256 * 4;
    const int64_t slots = L.tiles * (p.splits - 1) * m * kTileRows;
    p.exchange = p.splits > 1 && slots * 8 <= int64_t(kSyncBytes);
    p.workspace = p.splits == 1 ? 0
                  : p.exchange ? kSyncBytes
                               : kSyncBytes + size_t(p.splits) * m * L.tiles * kTileRows * 4;
    return p;
}

PlanInfo describe_mgemv(int64_t m, int64_t n, int64_t k, int bits) {
    const MgemvPlan p = plan_mgemv(m, n, k, bits);
    const Layout L(n, k, bits);
    return {p.waves, int(m), kTileRows, p.splits, p.gps, L.tiles * p.splits, p.splits > 1 && !p.exchange};
}

template <int MMAX, int ACT, int AF, int BITS>
static hipError_t launch_one(const MgemvArgs& a, const MgemvPlan& p, hipStream_t stream) {
    const Layout L(a.n, a.k, BITS);
    const dim3 grid(unsigned(L.tiles * p.splits)), block(unsigned(64 * p.waves));
    if (p.waves == 8) {
        // 17..32 groups per split (INT4 only): 8 waves of 4 chunks
        if constexpr (BITS == 4) mgemv_kernel<MMAX, ACT, 8, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a);
        else return hipErrorInvalidValue;
    } else {
        switch (p.cpw) {
            case 1: mgemv_kernel<MMAX, ACT, 4, 1, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
            case 2: mgemv_kernel<MMAX, ACT, 4, 2, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
            default: mgemv_kernel<MMAX, ACT, 4, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1 || p.exchange) return e;
    return launch_splitk_reduce(a.partials, p.splits, a.m, a.n, L.tiles * kTileRows, a.bias, a.y, a.ldy,
                                ACT, stream);
}

template <int MMAX, int ACT, int BITS>
static hipError_t launch_af(const MgemvArgs& a, const MgemvPlan& p, int act_fn, hipStream_t stream) {
    switch (act_fn) {
        case kActFnSwiglu: return launch_one<MMAX, ACT, kActFnSwiglu, BITS>(a, p, stream);
        case kActFnGeluTanh: return launch_one<MMAX, ACT, kActFnGeluTanh, BITS>(a, p, stream);
        default: return launch_one<MMAX, ACT, kActFnNone, BITS>(a, p, stream);
    }
}

template <int BITS>
static hipError_t launch_bits(const MgemvArgs& a, const MgemvPlan& p, int act, int act_fn, hipStream_t stream) {
    const bool bf = act == kActBf16;
    switch (p.mmax) {
        case 4: return bf ? launch_af<4, kActBf16, BITS>(a, p, act_fn, stream)
                          : launch_af<4, kActF16, BITS>(a, p, act_fn, stream);
        case 8: return bf ? launch_af<8, kActBf16, BITS>(a, p, act_fn, stream)
                          : launch_af<8, kActF16, BITS>(a, p, act_fn, stream);
        default: return bf ? launch_af<16, kActBf16, BITS>(a, p, act_fn, stream)
                           : launch_af<16, kActF16, BITS>(a, p, act_fn, stream);
    }
}

hipError_t launch_mgemv(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                        const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                        hipStream_t stream) {
    const MgemvPlan p = plan_mgemv(m, n, k, bits);
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
