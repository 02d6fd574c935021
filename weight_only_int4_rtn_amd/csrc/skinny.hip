// Mid-M forward (and any M): register-dequantized weights into MFMA.  Two
// kernels: skinny_direct_kernel (no fused activation; below) keeps the
// workgroup's whole x slice in LDS; skinny_kernel stages x per group:
//
// A workgroup of 4 waves owns 4 adjacent 16-row weight tiles (64 output
// columns), a block of up to 64 activation rows (MB 16-row blocks; the plan
// takes 16 or 32) and a K split of up to 16 groups (8 for MB > 2, half as
// many INT8 chunks).  Each wave first loads the x tiles of the first two
// groups, then the 1 KB chunks of its tile (one 128-bit load per lane each),
// 8 groups (4 with 32-row blocks) ahead of the group computed, so the first
// groups can start as soon as their own data lands (loads complete in issue
// order; x issued after the chunks would wait for them: measured 1-8 %
// slower).  Then per 128-column group:
//   1. the activation block's 128 columns, loaded into registers two groups
//      ahead, are staged in one of two LDS buffers (with a fused input
//      activation applied on the way);
//   2. each wave turns every word of its chunk into one MFMA B operand: the
//      chunk layout is the B-operand layout of v_mfma_f32_16x16x32_{bf16,f16}
//      (common.h), and each nibble pair becomes a packed pair of 16-bit
//      floats holding off + q exactly (off = 136 for bf16, 1032 for f16);
//   3. per 16-row m-subtile and k-step of 32, one MFMA adds x (off + q) and
//      a second one, with the same x fragment and a B operand of -off in
//      every element (exact in both 16-bit types), adds -off x: the
//      accumulator ends with the group's sum_k x q, which the wave multiplies
//      by the column's FP32 scale and adds into its FP32 totals.  The extra
//      MFMAs replace a per-row sum of x with its cross-lane reduction, whose
//      latency the few waves of this kernel could not hide (measured 15-31 %
//      faster for M 16-256).
// The weights never pass through LDS; x tiles are shared by the 4 waves.
// A K split finishes inside the launch: each split stores its FP32 sums in a
// workspace slot and the last to finish a tile adds them in split order, adds
// the bias in FP32 and rounds once (the split-K reduce kernel, reduce.hip,
// when the workspace header has no room for the tiles' counters).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

struct SkinnyArgs {
    const uint16_t* x;
    int64_t ldx, m;
    const uint8_t* packed;
    int64_t n, k;
    const uint16_t* bias;
    uint16_t* y;
    int64_t ldy;
    float* partials;  // [splits][m][tile_groups*64] when splits > 1 (reduce kernel)
    int splits, gps;
    int64_t tile_groups;
    // K split finished in-kernel: one counter per (tile group, row block) in
    // the workspace header, FP32 slots [splits][tile_groups][row blocks][16 MB x 64]
    unsigned* counters;
    float* slots;
    int in_kernel;
};

constexpr int kSkWaves = 4;
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kAStride = kGroup + 8;       // LDS row stride of the x tile (elements): 16 B pad

template <int ACT>
__device__ inline f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (ACT == kActBf16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// The end of a SKINNY launch for one workgroup: its FP32 sums (lane: rows
// 16 mb + 4 kq + i, i = 0..3, of column r of the wave's tile) stored with the
// bias, or a K split finished in the launch or through the reduce kernel.
// flag: one int of LDS that no wave reads or writes any more.
template <int MB, int ACT, int WAVES>
__device__ inline void skinny_finish(const SkinnyArgs& a, const f32x4_t (&tot)[MB], const int64_t tg,
                                     const int64_t mblk, const int split, int* const flag) {
    constexpr int BM = 16 * MB, COLS = 16 * WAVES;
    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t m0 = mblk * BM;
    const int64_t t = tg * WAVES + wave;
    const bool tile_ok = t < ceil_div(a.n, int64_t(kTileRows));
    const int64_t col = t * kTileRows + r;
    if (a.splits == 1) {
        if (tile_ok && col < a.n) {
            const float bv = a.bias ? to_f32<ACT>(a.bias[col]) : 0.0f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t row = m0 + mb * 16 + 4 * kq + i;
                    if (row < a.m) a.y[row * a.ldy + col] = from_f32<ACT>(tot[mb][i] + bv);
                }
        }
        return;
    }

    if (a.in_kernel) {
        // K split finished in this launch: every split stores its FP32 sums in
        // its slot, lane by lane as the registers hold them, written through
        // to the device's coherence point (SC1: the XCDs' L2s are not
        // coherent), and counts itself in the tile's counter; the split that
        // completes the count adds the slots in split order, 0 + s_0 + s_1 +
        // ... (its own sums from registers at their place: the reduce
        // kernel's order, so the same bits), clears the counter for the next
        // call and stores the outputs with the bias.  Nobody waits.
        const int64_t blocks = a.tile_groups * gridDim.y, tile = tg * gridDim.y + mblk;
        const int64_t slot_bytes = int64_t(BM) * COLS * 4;
        const __amdgpu_buffer_rsrc_t sl = buffer_rsrc(a.slots, int64_t(a.splits) * blocks * slot_bytes);
        const uint32_t lane_off = uint32_t((wave * MB * 64 + lane) * 16);
        auto slot_of = [&](int sp) { return uint32_t((int64_t(sp) * blocks + tile) * slot_bytes) + lane_off; };
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, tot[mb]), sl, slot_of(split) + mb * 1024,
                                                   0, kCoherent);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int* const last = flag;
        if (tid == 0) {
            const unsigned before =
                __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *last = before == unsigned(a.splits - 1);
            if (*last) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!*last) return;
        f32x4_t sum[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) sum[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // eight splits' sums in flight at a time
        for (int s0 = 0; s0 < a.splits; s0 += 8) {
            f32x4_t part[8][MB];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int sp = min(s0 + j, a.splits - 1);
                    part[j][mb] = sp == split ? tot[mb]
                                              : __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                                sl, slot_of(sp) + mb * 1024, 0,
                                                                                kCoherent));
                }
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    if (s0 + j < a.splits) sum[mb] += part[j][mb];
        }
        if (tile_ok && col < a.n) {
            const float bv = a.bias ? to_f32<ACT>(a.bias[col]) : 0.0f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t row = m0 + mb * 16 + 4 * kq + i;
                    if (row < a.m) a.y[row * a.ldy + col] = from_f32<ACT>(sum[mb][i] + bv);
                }
        }
        return;
    }

    // K split: store the FP32 partial sums; the split-K reduce kernel adds
    // them in split order, adds the bias and rounds (reduce.hip).
    if (!tile_ok) return;
    const int64_t npad = a.tile_groups * COLS;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = m0 + mb * 16 + 4 * kq + i;
            if (row < a.m) a.partials[(int64_t(split) * a.m + row) * npad + col] = tot[mb][i];
        }
}

// AF: activation fused into the x staging (ActFn; SwiGLU gate values sit k
// columns after the up values).  GMAX: most groups one workgroup covers (all
// of its chunks are held in registers, loaded a window ahead).  BITS: 4 (INT4 chunks) or 8 (INT8
// chunks, two 1 KB halves each).
template <int MB, int ACT, int AF, int GMAX, int BITS>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkinnyArgs a) {
    constexpr int BM = 16 * MB;
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    __shared__ __align__(16) uint16_t xa[2][BM * kAStride];

    const Layout L(a.n, a.k, BITS);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t tg = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t mblk = blockIdx.y;
    const int64_t m0 = mblk * BM;
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t t = tg * kSkWaves + wave;
    const bool tile_ok = t < L.tiles;
    const int64_t tt = tile_ok ? t : L.tiles - 1;  // loads stay in bounds; results unused
    const uint8_t* cbase = a.packed + (tt * L.groups + g0) * CB + lane * 16;
    const float* sbase = reinterpret_cast<const float*>(a.packed + L.scale_offset()) + (tt * L.groups + g0) * kTileRows + r;
    constexpr float off = code_offset<ACT, BITS>();
    // B operand of -off in every element (step 3 above)
    const uint32_t noff2 = uint32_t(from_f32<ACT>(-off)) * 0x00010001u;
    const uint4 bneg = make_uint4(noff2, noff2, noff2, noff2);

    // Every chunk and scale of the wave's groups (loaded below, right after
    // the first two groups' x).
    uint4 cw[GMAX][H];
    float sc[GMAX];

    // x of one group: rows m0 .. m0 + BM - 1, columns of the group; 16
    // threads per row, 8 columns each, MB passes (rows past M read row 0 and
    // are zeroed when staged).  Loaded into one of two register sets two
    // groups ahead, then activated and staged in one of two LDS buffers.
    uint4 xr[2][MB];
    uint4 xgate[AF == kActFnSwiglu ? 2 : 1][AF == kActFnSwiglu ? MB : 1];
    auto load_x = [&](int set, int gl) {
#pragma unroll
        for (int pass = 0; pass < MB; ++pass) {
            const int row = pass * 16 + (tid >> 4), piece = tid & 15;
            const bool on = m0 + row < a.m;
            const uint16_t* src = a.x + (on ? m0 + row : 0) * a.ldx + (g0 + gl) * kGroup + piece * 8;
            xr[set][pass] = *reinterpret_cast<const uint4*>(src);
            if constexpr (AF == kActFnSwiglu) xgate[set][pass] = *reinterpret_cast<const uint4*>(src + a.k);
        }
    };
    auto stage_x = [&](int set, int buf) {
#pragma unroll
        for (int pass = 0; pass < MB; ++pass) {
            const int row = pass * 16 + (tid >> 4), piece = tid & 15;
            uint4 v = xr[set][pass];
            if constexpr (AF != kActFnNone)
                v = activate8<ACT, AF>(v, xgate[AF == kActFnSwiglu ? set : 0][AF == kActFnSwiglu ? pass : 0]);
            if (m0 + row >= a.m) v = make_uint4(0u, 0u, 0u, 0u);
            *reinterpret_cast<uint4*>(&xa[buf][row * kAStride + piece * 8]) = v;
        }
    };

    f32x4_t tot[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_x(0, 0);
    if (ng > 1) load_x(1, 1);
    // keep the compiler from hoisting the chunk loads above the x loads
    __builtin_amdgcn_sched_barrier(0);
    // chunks in flight ahead of the group computed (the direct kernel's
    // window; issuing every chunk up front left a wave stalled at issue until
    // its stream had almost arrived: 8-11 % faster, 96 x 2048 x 16384 20.4 ->
    // 18.2 us, 16 x 16384 x 2048 with SwiGLU 14.8 -> 13.6)
    constexpr int SPF = MB == 1 ? 8 : 4;
    auto load_chunk = [&](int u) {
        const int gc = u < ng ? u : ng - 1;  // a valid chunk; unused when u >= ng
#pragma unroll
        for (int h = 0; h < H; ++h) cw[u][h] = load_stream16(cbase + int64_t(gc) * CB + h * kChunkBytes);
        sc[u] = sbase[int64_t(gc) * kTileRows];
    };
#pragma unroll
    for (int u = 0; u < (SPF < GMAX ? SPF : GMAX); ++u) load_chunk(u);
    stage_x(0, 0);
    __syncthreads();
#pragma unroll
    for (int gl = 0; gl < GMAX; ++gl) {
        if (gl + SPF < GMAX) load_chunk(gl + SPF);
        if (gl >= ng) continue;  // (not break: the loop stays fully unrolled, arrays in registers)
        const int buf = gl & 1;

        uint32_t words[4 * H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
            words[4 * h] = cw[gl][h].x;
            words[4 * h + 1] = cw[gl][h].y;
            words[4 * h + 2] = cw[gl][h].z;
            words[4 * h + 3] = cw[gl][h].w;
        }
        uint4 b01[2], b23[2];
        bpairs2<BITS, ACT>(words, 0, b01);
        bpairs2<BITS, ACT>(words, 2, b23);
        const uint4 b[4] = {b01[0], b01[1], b23[0], b23[1]};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* ap = &xa[buf][(mb * 16 + r) * kAStride + 8 * kq];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 av = *reinterpret_cast<const uint4*>(ap + 32 * s);
                acc = mfma16<ACT>(av, b[s], acc);
                acc = mfma16<ACT>(av, bneg, acc);
            }
            tot[mb][0] = fmaf(sc[gl], acc[0], tot[mb][0]);
            tot[mb][1] = fmaf(sc[gl], acc[1], tot[mb][1]);
            tot[mb][2] = fmaf(sc[gl], acc[2], tot[mb][2]);
            tot[mb][3] = fmaf(sc[gl], acc[3], tot[mb][3]);
        }
        // group gl + 1 into the other LDS buffer, last read in the previous
        // group, which ended with a barrier; then group gl + 2 into the
        // register set just staged from.  The loads go out after the staging:
        // the compiler's wait before the staging covers every load issued
        // before it, so loads issued earlier in this group would each cost a
        // full memory round trip per group.
        if (gl + 1 < ng) stage_x((gl + 1) & 1, buf ^ 1);
        if (gl + 2 < ng) load_x(gl & 1, gl + 2);
        __syncthreads();
    }

    skinny_finish<MB, ACT, kSkWaves>(a, tot, tg, mblk, split, reinterpret_cast<int*>(&xa[0][0]));
}

// A pair of groups' x fragments from LDS (the direct kernel's layout below;
// addr: this lane's byte address of the pair's first block, the second
// group's blocks 4 MB KB later): 8 MB reads in one asm block that also waits
// for them.  The compiler cannot tell LDS reads from the LDS the direct
// global-to-LDS loads still in flight write, so before a plain read it waits
// for every such load issued so far; these reads carry no such wait (the
// caller's own wait and barrier order them after their blocks' loads).  The
// outputs are early-clobber: no output may share the address register, which
// a read's returning data could otherwise overwrite before the block's later
// reads have issued.
template <int MB>
__device__ inline void read_pair(uint32_t addr, uint4 (&a0)[MB][4], uint4 (&a1)[MB][4]) {
    if constexpr (MB == 1) {
        asm volatile(
            "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
            "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0[0][0]), "=&v"(a0[0][1]), "=&v"(a0[0][2]), "=&v"(a0[0][3]), "=&v"(a1[0][0]), "=&v"(a1[0][1]),
              "=&v"(a1[0][2]), "=&v"(a1[0][3])
            : "v"(addr)
            : "memory");
    } else {
        static_assert(MB == 2, "m-subtiles");
        asm volatile(
            "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:1024\n\t"
            "ds_read_b128 %2, %16 offset:2048\n\tds_read_b128 %3, %16 offset:3072\n\t"
            "ds_read_b128 %4, %16 offset:4096\n\tds_read_b128 %5, %16 offset:5120\n\t"
            "ds_read_b128 %6, %16 offset:6144\n\tds_read_b128 %7, %16 offset:7168\n\t"
            "ds_read_b128 %8, %16 offset:8192\n\tds_read_b128 %9, %16 offset:9216\n\t"
            "ds_read_b128 %10, %16 offset:10240\n\tds_read_b128 %11, %16 offset:11264\n\t"
            "ds_read_b128 %12, %16 offset:12288\n\tds_read_b128 %13, %16 offset:13312\n\t"
            "ds_read_b128 %14, %16 offset:14336\n\tds_read_b128 %15, %16 offset:15360\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0[0][0]), "=&v"(a0[0][1]), "=&v"(a0[0][2]), "=&v"(a0[0][3]), "=&v"(a0[1][0]), "=&v"(a0[1][1]),
              "=&v"(a0[1][2]), "=&v"(a0[1][3]), "=&v"(a1[0][0]), "=&v"(a1[0][1]), "=&v"(a1[0][2]), "=&v"(a1[0][3]),
              "=&v"(a1[1][0]), "=&v"(a1[1][1]), "=&v"(a1[1][2]), "=&v"(a1[1][3])
            : "v"(addr)
            : "memory");
    }
}

// Without a fused activation: the workgroup's whole x slice in LDS.  4 MB
// waves (one 16-row weight tile each, 64 MB output columns) and up to 16
// groups of K (8 INT8 chunks), taken in pairs: two independent accumulator
// chains, interleaved (1-4 % faster than one group at a time).  Each wave
// loads one 1 KB x block per group (direct global-to-LDS loads), and the
// chunks and scales of its tile a window ahead of the pair being computed:
// a wave stalls at issue once the memory pipeline is full, so issuing
// every chunk up front kept each wave from computing until its whole stream
// had almost arrived (the window measured 3-10 % faster).  Two schedules:
//  * 16-row blocks: every x block first, then the chunks 8 groups ahead;
//    before pairs 0, 1, 2 and 4 each wave waits for its x blocks of groups
//    0-1, 2-3, 4-7 or 8-15 and a barrier makes everyone's visible;
//  * 32-row blocks (8 waves): a pair's two x blocks and two chunks go out
//    together, 2 pairs ahead; each pair waits for its own x blocks alone,
//    then a barrier, and its fragments are read by read_pair (6-8 % faster
//    than the first schedule here: 64 x 2048 x 16384 13.4 -> 12.5 us; 0-7 %
//    slower with 16-row blocks).
// The LDS holds x as MFMA A operands: block (group g, m-subtile mb, k-step
// s) holds lane l's 16 bytes, x[16 mb + (l & 15)][128 g + 32 s + 8 (l >> 4)
// .. + 7], at byte 16 l of block 4 MB g + 4 mb + s (linear: conflict-free
// reads).  Rows past M read zero through the buffer range.
template <int MB, int ACT, int GMAX, int BITS>
__global__ __launch_bounds__(256 * MB) void skinny_direct_kernel(SkinnyArgs a) {
    constexpr int WAVES = 4 * MB, NB = 4 * MB;  // NB: 1 KB x blocks per group, one per wave
    constexpr int BM = 16 * MB;
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    constexpr bool PAIRED = MB == 2;     // x loads in the window with the chunks
    constexpr int PF = MB == 1 ? 8 : 4;  // groups whose chunks are in flight ahead of the pair computed
    static_assert(GMAX % 2 == 0, "pairs");
    constexpr int NP = GMAX / 2, PP = PF / 2 < NP ? PF / 2 : NP;  // pairs; pairs ahead
    __shared__ __align__(16) uint8_t xl[GMAX * NB * 1024];

    const Layout L(a.n, a.k, BITS);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t tg = int64_t(blockIdx.x / unsigned(a.splits));
    const int64_t mblk = blockIdx.y;
    const int64_t m0 = mblk * BM;
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t t = tg * WAVES + wave;
    const int64_t tt = t < L.tiles ? t : L.tiles - 1;  // loads stay in bounds; results unused
    const uint8_t* cbase = a.packed + (tt * L.groups + g0) * CB + lane * 16;
    const float* sbase = reinterpret_cast<const float*>(a.packed + L.scale_offset()) + (tt * L.groups + g0) * kTileRows + r;
    constexpr float off = code_offset<ACT, BITS>();
    const uint32_t noff2 = uint32_t(from_f32<ACT>(-off)) * 0x00010001u;
    const uint4 bneg = make_uint4(noff2, noff2, noff2, noff2);

    // x blocks: this wave fills block `wave` (m-subtile wave / 4, k-step
    // wave % 4) of every group; groups past the split's end reload its last.
    const int64_t rows_valid = min<int64_t>(BM, a.m - m0);
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(a.x + m0 * a.ldx, rows_valid * a.ldx * 2);
    const uint32_t xoff = uint32_t((16 * (wave >> 2) + r) * a.ldx * 2 + (32 * (wave & 3) + 8 * kq) * 2);
    auto load_x = [&](int u) {
        const int gc = u < ng ? u : ng - 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_ptr_t)(xl + (u * NB + wave) * 1024), 16, xoff,
                                                 uniform(int((g0 + gc) * kGroup * 2)), 0, 0);
    };
    uint4 cw[GMAX][H];
    float sc[GMAX];
    auto load_chunk = [&](int u) {
        const int gc = u < ng ? u : ng - 1;
#pragma unroll
        for (int h = 0; h < H; ++h) cw[u][h] = load_stream16(cbase + int64_t(gc) * CB + h * kChunkBytes);
        sc[u] = sbase[int64_t(gc) * kTileRows];
    };
    // a pair's loads in the window (PAIRED: with its x blocks)
    constexpr int LP = (PAIRED ? 2 : 0) + 2 * (H + 1);  // loads per pair
    auto load_pair = [&](int p) {
        if constexpr (PAIRED) {
            load_x(2 * p);
            load_x(2 * p + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        load_chunk(2 * p);
        load_chunk(2 * p + 1);
        if constexpr (PAIRED) __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (!PAIRED) {
#pragma unroll
        for (int u = 0; u < GMAX; ++u) load_x(u);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < PP; ++p) load_pair(p);

    f32x4_t tot[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto decode = [&](int u, uint4 (&b)[4]) {
        uint32_t words[4 * H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
            words[4 * h] = cw[u][h].x;
            words[4 * h + 1] = cw[u][h].y;
            words[4 * h + 2] = cw[u][h].z;
            words[4 * h + 3] = cw[u][h].w;
        }
        uint4 b01[2], b23[2];
        bpairs2<BITS, ACT>(words, 0, b01);
        bpairs2<BITS, ACT>(words, 2, b23);
        b[0] = b01[0];
        b[1] = b01[1];
        b[2] = b23[0];
        b[3] = b23[1];
    };
    static_for<0, NP>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int g0 = 2 * j, g1 = 2 * j + 1;
        // this wave's x blocks of the groups about to be read have landed
        // (the loads issued after them may still be in flight), then
        // everyone's (a wave whose split ends early still takes part)
        constexpr int issued = j + PP < NP ? j + PP : NP;  // pairs in the window issued so far
        if constexpr (PAIRED) {
            wait_vm<2 * (H + 1) + (issued - j - 1) * LP>();
            lds_barrier();
        } else if constexpr (j == 0 || j == 1 || j == 2 || j == 4) {
            constexpr int end0 = j == 0 ? 2 : 4 * j;
            constexpr int end = end0 < GMAX ? end0 : GMAX;
            wait_vm<(GMAX - end) + issued * LP>();
            lds_barrier();
        }
        // then the pair PP ahead goes out, before this pair's work
        if constexpr (j + PP < NP) load_pair(j + PP);
        if (g0 >= ng) return;
        const bool two = g1 < ng;  // (else the second chain's sums are dropped)
        // the pair's x fragments first: their LDS latency passes during the
        // decode (3 % faster with 32-row blocks)
        uint4 av0[MB][4], av1[MB][4];
        if constexpr (PAIRED) {
            read_pair<MB>(uint32_t(reinterpret_cast<uintptr_t>(xl)) + uint32_t(g0 * NB * 1024 + lane * 16), av0, av1);
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    av0[mb][s] = *reinterpret_cast<const uint4*>(xl + ((g0 * NB + mb * 4 + s) * 1024) + lane * 16);
                    av1[mb][s] = *reinterpret_cast<const uint4*>(xl + ((g1 * NB + mb * 4 + s) * 1024) + lane * 16);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        uint4 b0[4], b1[4];
        decode(g0, b0);
        decode(g1, b1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                acc0 = mfma16<ACT>(av0[mb][s], b0[s], acc0);
                acc1 = mfma16<ACT>(av1[mb][s], b1[s], acc1);
                acc0 = mfma16<ACT>(av0[mb][s], bneg, acc0);
                acc1 = mfma16<ACT>(av1[mb][s], bneg, acc1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[mb][i] = fmaf(sc[g0], acc0[i], tot[mb][i]);
            if (two) {
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[mb][i] = fmaf(sc[g1], acc1[i], tot[mb][i]);
            }
        }
    });
    // (the finish writes its flag only after a barrier all waves reach after
    // their last read of the slice)
    skinny_finish<MB, ACT, WAVES>(a, tot, tg, mblk, split, reinterpret_cast<int*>(xl));
}

namespace {

// The plan for one kernel: 16-row m-subtiles per workgroup (mb) and the x
// slice whole in LDS (direct) or staged per group.
SkinnyPlan make_skinny_plan(int64_t m, const Layout& L, int mb, bool direct) {
    SkinnyPlan p{};
    p.mb = mb;
    const int64_t bm = 16 * p.mb;
    p.mblocks = ceil_div(m, bm);
    // the direct kernel: 4 waves per 16-row block (8 tiles share each x
    // block of a 32-row block)
    p.direct = direct;
    p.waves = direct ? 4 * mb : kSkWaves;
    const int64_t cols = 16 * p.waves;
    p.tile_groups = ceil_div(L.tiles, int64_t(p.waves));
    // A workgroup holds all of its chunks in registers: up to 16 groups with
    // one or two 16-row m-subtiles, 8 with more.  Split K beyond that, and
    // further (halving the groups per workgroup) while fewer than 256
    // workgroups would run (measured: that beats the cost of the reduce
    // launch a split adds).
    const int64_t minwg = 256;
    // (INT8 chunks take twice the registers: half the groups)
    const int64_t cap = (p.mb <= 2 ? 16 : 8) / (L.cb == kChunkBytes8 ? 2 : 1);
    const int64_t base = p.tile_groups * p.mblocks;
    int64_t gps = L.groups < cap ? L.groups : cap;
    // INT4 layers of <= 8 M weights: at most 8 groups per split, and not
    // below 4 (MI355X, us, M x K x N: 128 x 4096 x 1024 in four splits of 8
    // 9.5 vs two of 16 12.0; 64 x 4096 x 2048 8.1 vs 9.0; 64 x 8192 x 1024
    // 9.1 vs 9.7; 16 x 4096 x 1024 in splits of 4 6.7 vs 2 8.8; from 8 to 4
    // groups per split slower: 50 x 4096 x 1024 8.1 vs 7.3)
    const bool small = L.cb == kChunkBytes && L.tiles * kTileRows * L.groups * kGroup <= (int64_t(8) << 20);
    if (small && gps > 8) gps = 8;
    const int64_t floor_gps = small ? 4 : 2;
    while (gps > floor_gps && base * ceil_div(L.groups, gps) < minwg) gps = ceil_div(gps, 2);
    p.gps = int(gps);
    p.gmax = gps <= 4 ? 4 : gps <= 8 ? 8 : 16;
    p.splits = int(ceil_div(L.groups, gps));
    // A split finishes inside the launch (tile counters in the workspace
    // header, slots after it) where the counters and the slots' 32-bit
    // offsets fit: 7-14 % faster than through the reduce kernel's launch
    // (16 x 16384 x 2048: 13.8 -> 11.9 us; 64 x 16384 x 2048: 20.4 -> 17.9;
    // 50 x 4096 x 1024: 9.2 -> 8.2).
    const int64_t blocks = p.tile_groups * p.mblocks;
    const int64_t slot_bytes = int64_t(p.splits) * blocks * bm * cols * 4;
    p.in_kernel = p.splits > 1 && blocks <= int64_t(kSyncBytes / 4) && slot_bytes < (int64_t(1) << 31);
    p.workspace = p.splits == 1 ? 0
                  : p.in_kernel ? kSyncBytes + size_t(slot_bytes)
                                : kSyncBytes + size_t(p.splits) * m * p.tile_groups * cols * 4;
    return p;
}

}  // namespace

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int bits, int act_fn) {
    const Layout L(n, k, bits);
    // Row blocks: these launches are latency-bound, so more and shorter
    // workgroups win while the weights are small enough that reading them
    // once per 16-row block stays cheap (from L2); larger layers take 32-row
    // blocks.  Measured (MI355X, M 20..127): layers of <= 8 M weights run
    // 1.3-1.8x faster with 16-row blocks than with 64-row blocks, layers of
    // 33.5 M weights 10-20 % faster with 32-row blocks than with 16 or 64.
    const bool small = n * k <= (int64_t(8) << 20);
    const int mb = m <= 16 || small ? 1 : 2;
    // Without a fused activation the direct kernel (x slice whole in LDS)
    // where it measured faster (MI355X, bf16): 16-row blocks up to M = 64,
    // 7-15 % (16 x 16384 x 2048: 11.9 -> 10.5 us; 16 x 2048 x 16384: 9.6 ->
    // 8.2; 50 x 4096 x 1024: 8.0 -> 7.5; 64 x 1024 x 4096: 5.4 -> 4.9), not
    // beyond (256 x 1024 x 4096: 9.1 -> 10.0); 32-row blocks in one round of
    // workgroups (at most one per CU: 128 KB of LDS) with at most 8 K
    // splits (64 x 2048 x 16384: 15.9 -> 12.7; 64 x 16384 x 2048: 18.0 ->
    // 17.3; 50 x 16384 x 2048: 17.8 -> 16.7); in more rounds or with 16
    // splits they ran 4-45 % slower (32 x 16384 x 2048: 14.6 -> 15.2; 96 x
    // 2048 x 16384: 20.4 -> 27.0).
    if (act_fn == kActFnNone) {
        if (mb == 1 && m <= 64) return make_skinny_plan(m, L, 1, true);
        if (mb == 2) {
            const SkinnyPlan d = make_skinny_plan(m, L, 2, true);
            if (d.splits <= 8 && d.tile_groups * d.mblocks * d.splits <= 256) return d;
        }
    }
    return make_skinny_plan(m, L, mb, false);
}

PlanInfo describe_skinny(int64_t m, int64_t n, int64_t k, int bits, int act_fn) {
    const SkinnyPlan p = plan_skinny(m, n, k, bits, act_fn);
    return {p.waves, 16 * p.mb, 16 * p.waves, p.splits, p.gps, p.tile_groups * p.splits * p.mblocks,
            p.splits > 1 && !p.in_kernel};
}

template <int MB, int ACT, int AF, int BITS>
static hipError_t launch_one(const SkinnyArgs& a, const SkinnyPlan& p, hipStream_t stream) {
    dim3 grid(unsigned(p.tile_groups * p.splits), unsigned(p.mblocks));
    // the plan keeps the register footprint GMAX * BITS / 4 chunks <= 16, and
    // <= 8 for MB > 2
    constexpr int kMaxRegChunks = MB <= 2 ? 16 : 8;
    if (p.direct) {
        // (the plan takes it only without a fused activation, MB <= 2)
        if constexpr (AF == kActFnNone && MB <= 2) {
            const dim3 block(unsigned(256 * MB));
            if (p.gmax == 4) skinny_direct_kernel<MB, ACT, 4, BITS><<<grid, block, 0, stream>>>(a);
            else if (p.gmax == 8) skinny_direct_kernel<MB, ACT, 8, BITS><<<grid, block, 0, stream>>>(a);
            else if constexpr (16 * BITS / 4 <= kMaxRegChunks) skinny_direct_kernel<MB, ACT, 16, BITS><<<grid, block, 0, stream>>>(a);
            else return hipErrorInvalidValue;
        } else {
            return hipErrorInvalidValue;
        }
    } else if (p.gmax == 4) {
        if constexpr (4 * BITS / 4 <= kMaxRegChunks) skinny_kernel<MB, ACT, AF, 4, BITS><<<grid, dim3(kSkThreads), 0, stream>>>(a);
        else return hipErrorInvalidValue;
    } else if (p.gmax == 8) {
        if constexpr (8 * BITS / 4 <= kMaxRegChunks) skinny_kernel<MB, ACT, AF, 8, BITS><<<grid, dim3(kSkThreads), 0, stream>>>(a);
        else return hipErrorInvalidValue;
    } else {
        if constexpr (16 * BITS / 4 <= kMaxRegChunks) skinny_kernel<MB, ACT, AF, 16, BITS><<<grid, dim3(kSkThreads), 0, stream>>>(a);
        else return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1 || p.in_kernel) return e;
    return launch_splitk_reduce(a.partials, p.splits, a.m, a.n, p.tile_groups * 16 * p.waves, a.bias, a.y, a.ldy,
                                ACT, stream);
}

template <int MB, int ACT, int BITS>
static hipError_t launch_af(const SkinnyArgs& a, const SkinnyPlan& p, int act_fn, hipStream_t stream) {
    switch (act_fn) {
        case kActFnSwiglu: return launch_one<MB, ACT, kActFnSwiglu, BITS>(a, p, stream);
        case kActFnGeluTanh: return launch_one<MB, ACT, kActFnGeluTanh, BITS>(a, p, stream);
        default: return launch_one<MB, ACT, kActFnNone, BITS>(a, p, stream);
    }
}

template <int MB>
static hipError_t launch_mb(const SkinnyArgs& a, const SkinnyPlan& p, int act, int act_fn, int bits,
                            hipStream_t stream) {
    const bool bf = act == kActBf16;
    if (bits == 8)
        return bf ? launch_af<MB, kActBf16, 8>(a, p, act_fn, stream) : launch_af<MB, kActF16, 8>(a, p, act_fn, stream);
    return bf ? launch_af<MB, kActBf16, 4>(a, p, act_fn, stream) : launch_af<MB, kActF16, 4>(a, p, act_fn, stream);
}

hipError_t launch_skinny(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                         const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                         hipStream_t stream) {
    const SkinnyPlan p = plan_skinny(m, n, k, bits, act_fn);
    SkinnyArgs a;
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
    a.splits = p.splits;
    a.gps = p.gps;
    a.tile_groups = p.tile_groups;
    a.counters = static_cast<unsigned*>(workspace);
    a.slots = a.partials;
    a.in_kernel = p.in_kernel;
    switch (p.mb) {
        case 1: return launch_mb<1>(a, p, act, act_fn, bits, stream);
        case 2: return launch_mb<2>(a, p, act, act_fn, bits, stream);
        case 3: return launch_mb<3>(a, p, act, act_fn, bits, stream);
        default: return launch_mb<4>(a, p, act, act_fn, bits, stream);
    }
}

}  // namespace w4a16
