// Small-M forward (M <= 4): the decode / one-action-chunk regime, where the
// layer is a stream over the packed weight and HBM bandwidth is the bound.
//
// Work decomposition: a workgroup of WAVES waves owns one 16-row tile and a
// contiguous range of 128-column groups (a K split).  Wave w takes groups
// w, w + WAVES, ... of that range, so the waves read adjacent 1 KB chunks.
// Each lane loads its 16 bytes of a chunk with one 128-bit load (a wave reads
// the whole 1 KB chunk in one instruction), turns each pair of nibbles into a
// packed pair of 16-bit floats with one shift and one v_and_or, and multiplies
// them into the activations with v_dot2 (FP32 accumulation).
//
// Latency: each thread first loads its part of the x slice, then the chunks
// of its wave (nontemporal loads: the weights are read once; beyond 4 chunks
// per wave, 4 ahead of the one computed), then stages x in LDS.  Loads
// complete in issue order, so the staging waits only for x and every chunk is
// used as soon as it lands: the nibble arithmetic overlaps the weight stream
// instead of trailing it.
//
// The packed pairs hold 136 + q (bf16) or 1032 + q (f16) exactly; the offset
// is removed once per group with the sum of the lane's 32 activations, which
// the workgroup computes while it stages x:
//     sum_k x_k q_k = sum_k x_k (off + q_k) - off * sum_k x_k.
// The group's FP32 scale is applied once per group:  acc += s * that.
//
// Reduction: the 4 lanes that share a row (L, L+16, L+32, L+48) are summed
// with two cross-lane exchanges and the waves through LDS in a fixed order.
// Without a K split the workgroup then adds the bias in FP32 and rounds once
// to the output dtype.  A K longer than one workgroup covers (32 groups) is
// split over workgroups whose row sums meet in a fixed binary tree of
// exchange slots: at each node the two children's sums are added (FP32
// addition is commutative, so the result does not depend on which child
// arrives first); the root adds the bias and rounds.  One launch, no
// floating-point atomics, reproducible results.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

struct GemvArgs {
    const uint16_t* x;
    int64_t ldx;
    const uint8_t* packed;
    int64_t n, k;
    const uint16_t* bias;
    uint16_t* y;
    int64_t ldy;
    unsigned long long* slots;  // [tiles][splits - 1][M * 16] exchange slots, zero before and after a call
    float* partials;            // [splits][M][tiles * 16] when the slots do not fit: split-K reduce kernel
    int splits;
    int gps;                    // groups per split
    int exchange;               // splits > 1: finish through the slots (else through partials)
};

// AF: activation fused into the x staging (ActFn); for SwiGLU the x rows
// hold [up | gate] and the gate values sit k columns after the up values.
// BITS: 4 (INT4 chunks) or 8 (INT8 chunks, two 1 KB halves per chunk).
template <int M, int ACT, int WAVES, int CPW, int AF, int BITS>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(GemvArgs a) {
    constexpr int THREADS = 64 * WAVES;
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    // 16-byte x loads per thread while staging: the slice is M rows of at
    // most WAVES * CPW groups of 128 columns, M * CPW / 4 loads per thread.
    constexpr int kXRegs = (M * CPW + 3) / 4;
    extern __shared__ __align__(16) unsigned char smem[];
    // the x pointer in the first batch of kernel-argument loads (else the
    // compiler fetches it separately, just before the x loads: one more
    // scalar-memory round trip before any load is issued)
    asm volatile("" ::"s"(a.x));
    const Layout L(a.n, a.k, BITS);
    // no integer division before the first load when K is not split (the
    // common decode case): it sits on every workgroup's path to its loads
    int split = 0;
    int64_t t = blockIdx.x;
    if (a.splits > 1) {
        split = int(blockIdx.x % unsigned(a.splits));
        t = int64_t(blockIdx.x / unsigned(a.splits));
    }
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));
    const int klen = ng * kGroup;

    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                              // [M][klen]
    float* xsum = reinterpret_cast<float*>(smem + size_t(M) * a.gps * kGroup * 2);   // [M][ng][4]
    float* red = xsum + M * a.gps * 4;                                             // [WAVES][M][16]

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;

    // Every chunk of the wave (CPW of them) is loaded before any is used.
    // The loads are unconditional straight-line code (clamped addresses), so
    // the compiler's wait counts stay exact: each use waits for its own load.
    uint4 cw[CPW][H];
    float sc[CPW];

    // x slice first (loads complete in issue order, so the weight loads
    // issued next never delay the staging), then the first weight batch.
    // The plan keeps M * klen / 8 <= kXRegs * THREADS.
    const int per_row = klen / 8;  // multiple of 16
    const int total = M * per_row;  // <= 2048: M <= 4 rows of <= 4096 columns
    const float inv_row = 1.0f / float(per_row);
    // zero-initialised so every register has a value on every path out of
    // the load loop (the compiler then keeps all x loads in flight together)
    uint4 xv[kXRegs];
#pragma unroll
    for (int j = 0; j < kXRegs; ++j) xv[j] = make_uint4(0u, 0u, 0u, 0u);
    uint4 xgate[AF == kActFnSwiglu ? kXRegs : 1];
#pragma unroll
    for (int j = 0; j < kXRegs; ++j) {
        if (j * THREADS >= total) break;
        const int i = j * THREADS + tid;
        const int ic = i < total ? i : total - 1;
        const int m = M == 1 ? 0 : div_small(ic, inv_row), c = ic - m * per_row;
        const uint16_t* src = a.x + m * a.ldx + g0 * kGroup + c * 8;
        xv[j] = *reinterpret_cast<const uint4*>(src);
        if constexpr (AF == kActFnSwiglu) xgate[j] = *reinterpret_cast<const uint4*>(src + a.k);
    }
    // keep the compiler from hoisting the weight loads (and their address
    // arithmetic) above the x loads
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* cbase = a.packed + (t * L.groups + g0) * CB + lane * 16;
    const float* sbase = reinterpret_cast<const float*>(a.packed + L.scale_offset()) + (t * L.groups + g0) * kTileRows + r;
    // M = 1: the split's chunks and scales through buffer resources, so a
    // chunk's address is a scalar offset plus the lane's 16 bytes (measured
    // faster at M = 1 only; larger M keep the flat loads)
    const __amdgpu_buffer_rsrc_t cres = buffer_rsrc(a.packed + (t * L.groups + g0) * CB, int64_t(ng) * CB);
    const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(
        a.packed + L.scale_offset() + (t * L.groups + g0) * kChunkScaleBytes, int64_t(ng) * kChunkScaleBytes);

    // A wave of more than 4 chunks issues 4 up front and each further one
    // while computing the chunk 4 before it: a wave stalls at issue once the
    // memory pipeline is full, so with every chunk issued up front it would
    // compute nothing until its stream had almost arrived (M = 1, 8 chunks
    // per wave: 16384 x 2048 6.47 -> 5.91 us; windows of 2, 3 and 6 chunks
    // 6.08-6.27).  INT8 chunks are twice as long: a window of 2 (16384 x
    // 2048 in two splits of 8 x 8 chunks: 8.3 us, 8.65 with a window of 4,
    // 9.1 in eight splits of 4 x 4 all up front).
    constexpr int PF = CPW < (BITS == 8 ? 2 : 4) ? CPW : (BITS == 8 ? 2 : 4);
    auto load_chunk = [&](int u) {
        const int gl = wave + u * WAVES;
        const int gc = gl < ng ? gl : ng - 1;  // a valid chunk; unused when gl >= ng
        if constexpr (M == 1) {
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(cres, lane * 16 + h * kChunkBytes, uniform(gc * CB),
                                                                     kBufNontemporal);
                cw[u][h] = make_uint4(v[0], v[1], v[2], v[3]);
            }
            sc[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   sres, r * 4, uniform(gc * kChunkScaleBytes), kBufNontemporal));
        } else {
#pragma unroll
            for (int h = 0; h < H; ++h) cw[u][h] = load_stream16(cbase + int64_t(gc) * CB + h * kChunkBytes);
            sc[u] = sbase[int64_t(gc) * kTileRows];
        }
        // Issue each chunk's scale right after its codes.  Left alone, the
        // compiler issues all code loads, then all scale loads; loads
        // complete in order, so the wait for chunk 0's scale then waits for
        // every chunk and the products of the later chunks no longer overlap
        // the stream.
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) load_chunk(u);

    // Stage x into LDS and sum each lane-quarter's 32 activations of every
    // group: block b = 4s + kq of a group holds columns 32s + 8kq .. +7, so a
    // quarter sum combines blocks kq, kq+4, kq+8, kq+12 (lanes 4 and 8 apart;
    // whole 16-lane segments are in or out of range together).
#pragma unroll
    for (int j = 0; j < kXRegs; ++j) {
        if (j * THREADS >= total) break;
        const int i = j * THREADS + tid;
        const bool on = i < total;
        const int m = (M == 1 || !on) ? 0 : div_small(i, inv_row), c = on ? i - m * per_row : 0;
        if constexpr (AF != kActFnNone) xv[j] = activate8<ACT, AF>(xv[j], xgate[AF == kActFnSwiglu ? j : 0]);
        if (on) *reinterpret_cast<uint4*>(xs + m * klen + c * 8) = xv[j];
        if (!on) xv[j] = make_uint4(0u, 0u, 0u, 0u);
        float s = sum8<ACT>(xv[j]);
        s += lane_xor<4>(s);
        s += lane_xor<8>(s);
        const int wb = c & 15;
        if (on && wb < 4) xsum[(m * ng + (c >> 4)) * 4 + wb] = s;
    }
    lds_barrier();

    constexpr float off = code_offset<ACT, BITS>();
    float tot[M];
#pragma unroll
    for (int m = 0; m < M; ++m) tot[m] = 0.0f;

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
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint16_t* xp = xs + m * klen + gl * kGroup + 8 * kq;
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < 4; s += 2) {
                    uint4 bp[2];
                    bpairs2<BITS, ACT>(words, s, bp);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint4 xq = *reinterpret_cast<const uint4*>(xp + 32 * (s + h));
                        acc = dot2<ACT>(bp[h].x, xq.x, acc);
                        acc = dot2<ACT>(bp[h].y, xq.y, acc);
                        acc = dot2<ACT>(bp[h].z, xq.z, acc);
                        acc = dot2<ACT>(bp[h].w, xq.w, acc);
                    }
                }
                acc = fmaf(-off, xsum[(m * ng + gl) * 4 + kq], acc);
                tot[m] = fmaf(scale, acc, tot[m]);
            }
        }
    }

    // Rows: sum the 4 lane-quarters, then the waves.
#pragma unroll
    for (int m = 0; m < M; ++m) {
        tot[m] += lane_xor<16>(tot[m]);
        tot[m] = sum_xor32(tot[m]);
        if (lane < 16) red[(wave * M + m) * 16 + lane] = tot[m];
    }
    lds_barrier();
    const bool out_thread = tid < M * 16;
    const int om = tid >> 4, orow = tid & 15;
    float v = 0.0f;
    if (out_thread) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[(w * M + om) * 16 + orow];
    }
    const int64_t ncol = t * kTileRows + orow;
    if (a.splits > 1 && !a.exchange) {
        if (out_thread) a.partials[(int64_t(split) * M + om) * (L.tiles * kTileRows) + ncol] = v;
        return;
    }
    if (a.splits > 1) {
        // Binary tree over the splits: leaf i = split i, node j of a level
        // joins children 2j and 2j + 1 of the level below (an odd last child
        // moves up alone).  Each output thread swaps its sum, tagged, into
        // its row's slot of the node with one device-scope 64-bit atomic
        // exchange.  An empty slot (tag 0) means the sibling has not arrived:
        // this thread is done.  Otherwise the old value is the sibling's sum:
        // the thread clears the slot for the next call, adds, and climbs.
        // The sums travel inside the atomics, so no fence is needed, and no
        // thread ever waits for another.
        if (!out_thread) return;
        int node_base = 0, idx = split, width = a.splits;
        while (width > 1) {
            if (!((width & 1) && idx == width - 1)) {
                unsigned long long* slot =
                    a.slots + (t * (a.splits - 1) + node_base + (idx >> 1)) * (M * kTileRows) + tid;
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
    if (out_thread && ncol < a.n) {
        if (a.bias) v += to_f32<ACT>(a.bias[ncol]);
        a.y[om * a.ldy + ncol] = from_f32<ACT>(v);
    }
}

// --- planning ---------------------------------------------------------------
//
// One row tile per workgroup.  Up to 16 groups per split: 4 waves of at most
// 4 chunks.  Beyond that 8 waves: at M = 1 a split holds up to 64 groups (8
// chunks per wave), or 128 (16) when the row tiles alone make 256
// workgroups, chunks issued 4 ahead (above); at M = 2-4 up to 32 groups (4
// chunks per wave, all up front).  Measured at M = 1 (MI355X, graph replay,
// us): 16384 x 2048 (128 tiles) in two splits of 64 groups 5.91 against
// four of 32 6.54 and one of 128 on 128 workgroups 6.93; 16384 x 4096 (256
// tiles) unsplit 8.28 against two splits 8.87 and four 9.2; 32768 x 1024
// in four splits of 64 6.38 against eight of 32 7.06.  INT8 chunks are
// twice as long: 4 waves of at most 4 of them, but at M = 1 splits of up to
// 64 groups on 8 waves with a window of 2 chunks (16384 x 2048: 8.3 us
// against 9.1 in eight splits of 16; 32768 x 1024 8.7 vs 9.6; 16384 x 4096
// 13.5 vs 14.8).
//
// Splitting only to fill the chip costs more than it gains: the exchange
// adds a device round trip per tree level (about 0.45 us each, measured),
// while a tile's chunks are all in flight at once anyway.  Nor do two
// workgroups per tile, one per 8-row half of every chunk, pay: measured
// slower than a K split on every shape tried (the two halves of a chunk are
// then read at different times from different XCDs).  The exchange slots
// live in the workspace's zero header; a launch whose tree does not fit
// there stores partial sums for the split-K reduce kernel instead.

GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k, int bits) {
    GemvPlan p{};
    const Layout L(n, k, bits);
    const int64_t G = L.groups;
    const int mm = int(m);
    const int64_t cap = bits == 8 ? (mm == 1 ? 8 * 8 : 4 * 4) : mm > 1 ? 8 * 4 : L.tiles >= 256 ? 8 * 16 : 8 * 8;
    const int64_t gps = G < cap ? G : cap;
    p.gps = int(gps);
    p.splits = int(ceil_div(G, gps));
    p.waves = gps > 16 ? 8 : 4;
    const int64_t per_wave = ceil_div(gps, p.waves);
    p.cpw = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : per_wave <= 8 ? 8 : 16;
    p.lds = size_t(mm) * gps * kGroup * 2 + size_t(mm) * gps * 4 * 4 + size_t(p.waves) * mm * 16 * 4;
    const int64_t slots = L.tiles * (p.splits - 1) * mm * kTileRows;
    p.exchange = p.splits > 1 && slots * 8 <= int64_t(kSyncBytes);
    p.workspace = p.splits == 1 ? 0
                  : p.exchange ? kSyncBytes
                               : kSyncBytes + size_t(p.splits) * mm * L.tiles * kTileRows * 4;
    return p;
}

PlanInfo describe_gemv(int64_t m, int64_t n, int64_t k, int bits) {
    const GemvPlan p = plan_gemv(m, n, k, bits);
    const Layout L(n, k, bits);
    return {p.waves, int(m), kTileRows, p.splits, p.gps, L.tiles * p.splits, p.splits > 1 && !p.exchange};
}

template <int M, int ACT, int AF, int BITS>
static hipError_t launch_one(const GemvArgs& a, const GemvPlan& p, hipStream_t stream) {
    const Layout L(a.n, a.k, BITS);
    const dim3 grid(unsigned(L.tiles * p.splits)), block(unsigned(64 * p.waves));
    if (p.waves == 8) {
        // 17..128 groups per split: INT4 8 waves of 4 chunks, or at M = 1 of
        // 8 or 16; INT8 only at M = 1, 8 waves of 4 or 8 chunks
        if constexpr (BITS == 8 && M == 1) {
            if (p.cpw == 8) gemv_kernel<M, ACT, 8, 8, AF, BITS><<<grid, block, p.lds, stream>>>(a);
            else if (p.cpw == 4) gemv_kernel<M, ACT, 8, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a);
            else return hipErrorInvalidValue;
        } else if constexpr (BITS == 4) {
            if constexpr (M == 1) {
                if (p.cpw == 16) gemv_kernel<M, ACT, 8, 16, AF, BITS><<<grid, block, p.lds, stream>>>(a);
                else if (p.cpw == 8) gemv_kernel<M, ACT, 8, 8, AF, BITS><<<grid, block, p.lds, stream>>>(a);
                else gemv_kernel<M, ACT, 8, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a);
            } else {
                if (p.cpw != 4) return hipErrorInvalidValue;
                gemv_kernel<M, ACT, 8, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a);
            }
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        switch (p.cpw) {
            case 1: gemv_kernel<M, ACT, 4, 1, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
            case 2: gemv_kernel<M, ACT, 4, 2, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
            default: gemv_kernel<M, ACT, 4, 4, AF, BITS><<<grid, block, p.lds, stream>>>(a); break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1 || p.exchange) return e;
    return launch_splitk_reduce(a.partials, p.splits, M, a.n, L.tiles * kTileRows, a.bias, a.y, a.ldy, ACT,
                                stream);
}

template <int M, int ACT, int BITS>
static hipError_t launch_af(const GemvArgs& a, const GemvPlan& p, int act_fn, hipStream_t stream) {
    switch (act_fn) {
        case kActFnSwiglu: return launch_one<M, ACT, kActFnSwiglu, BITS>(a, p, stream);
        case kActFnGeluTanh: return launch_one<M, ACT, kActFnGeluTanh, BITS>(a, p, stream);
        default: return launch_one<M, ACT, kActFnNone, BITS>(a, p, stream);
    }
}

template <int M>
static hipError_t launch_m(const GemvArgs& a, const GemvPlan& p, int act, int act_fn, int bits,
                           hipStream_t stream) {
    const bool bf = act == kActBf16;
    if (bits == 8)
        return bf ? launch_af<M, kActBf16, 8>(a, p, act_fn, stream) : launch_af<M, kActF16, 8>(a, p, act_fn, stream);
    return bf ? launch_af<M, kActBf16, 4>(a, p, act_fn, stream) : launch_af<M, kActF16, 4>(a, p, act_fn, stream);
}

hipError_t launch_gemv(const void* x, int act, int act_fn, int bits, int64_t m, int64_t k, int64_t ldx,
                       const void* packed, int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream) {
    const GemvPlan p = plan_gemv(m, n, k, bits);
    GemvArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
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
    switch (m) {
        case 1: return launch_m<1>(a, p, act, act_fn, bits, stream);
        case 2: return launch_m<2>(a, p, act, act_fn, bits, stream);
        case 3: return launch_m<3>(a, p, act, act_fn, bits, stream);
        default: return launch_m<4>(a, p, act, act_fn, bits, stream);
    }
}

}  // namespace w4a16
