// Small-M forward (M <= 4): the decode / one-action-chunk regime, where the
// layer is a stream over the packed weight and HBM bandwidth is the bound.
//
// Work decomposition: a workgroup of 4 waves owns one 16-row tile and a
// contiguous range of 128-column groups (a K split).  Wave w takes groups
// w, w+4, ... of that range, so the 4 waves read adjacent 1 KB chunks.  Each
// lane loads its 16 bytes of a chunk with one 128-bit load (a wave reads the
// whole 1 KB chunk in one instruction), turns each pair of nibbles into a
// packed pair of 16-bit floats with one shift and one and-or, and multiplies
// them into the activations with v_dot2 (FP32 accumulation).
//
// The packed pairs hold 136 + q (bf16) or 1032 + q (f16) exactly; the offset
// is removed once per group with the sum of the lane's 32 activations, which
// the workgroup computes while it stages its slice of x into LDS:
//     sum_k x_k q_k = sum_k x_k (off + q_k) - off * sum_k x_k.
// The group's FP32 scale is applied once per group:  acc += s * that.
//
// Reduction: the 4 lanes that share a row (L, L+16, L+32, L+48) are summed
// with two cross-lane exchanges, the 4 waves through LDS in a fixed order,
// and K splits through a workspace: every workgroup writes its partial row
// sums, and the last one to arrive at the tile (an integer counter) adds the
// partials in split order, adds the bias in FP32 and rounds once to the
// output dtype.  No floating-point atomics, so results are reproducible.
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
    float* partials;     // [tiles of the launch][splits][M][16]
    uint32_t* counters;  // [tiles of the launch]
    int64_t t0;          // first tile of the launch
    int splits;
    int gps;             // groups per split
};

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGemvBatch = 4;  // chunk loads a wave keeps in flight

template <int M, int ACT>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Layout L(a.n, a.k);
    const int split = int(blockIdx.x % unsigned(a.splits));
    const int64_t tl = int64_t(blockIdx.x / unsigned(a.splits));  // tile within the launch
    const int64_t t = a.t0 + tl;
    const int64_t g0 = int64_t(split) * a.gps;
    const int ng = int(min<int64_t>(a.gps, L.groups - g0));
    const int klen = ng * kGroup;

    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                             // [M][klen]
    float* xsum = reinterpret_cast<float*>(smem + size_t(M) * a.gps * kGroup * 2);  // [M][ng][4]
    float* red = xsum + M * a.gps * 4;                                            // [waves][M][16]

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kq = lane >> 4;

    // Stage x[:, g0*128 : g0*128 + klen) into LDS, 16 bytes per thread and step.
    {
        const int per_row = klen / 8;
        for (int i = tid; i < M * per_row; i += kGemvThreads) {
            const int m = i / per_row, c = i - m * per_row;
            const uint4 v = *reinterpret_cast<const uint4*>(a.x + m * a.ldx + g0 * kGroup + c * 8);
            *reinterpret_cast<uint4*>(xs + m * klen + c * 8) = v;
        }
    }
    __syncthreads();
    // Sums of each lane-quarter's 32 activations per group: columns
    // 32s + 8kq + j, s = 0..3, j = 0..7.
    for (int i = tid; i < M * ng * 4; i += kGemvThreads) {
        const int m = i / (ng * 4), rem = i - m * ng * 4, gl = rem >> 2, q4 = rem & 3;
        const uint16_t* p = xs + m * klen + gl * kGroup + 8 * q4;
        float s = 0.0f;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int j = 0; j < 8; ++j) s += to_f32<ACT>(p[32 * s4 + j]);
        xsum[i] = s;
    }
    __syncthreads();

    const uint8_t* cbase = a.packed + (t * L.groups + g0) * kChunkBytes + lane * 16;
    const float* sbase = reinterpret_cast<const float*>(a.packed + L.scale_offset()) + (t * L.groups + g0) * kTileRows + r;
    constexpr float off = code_offset<ACT>();

    float tot[M];
#pragma unroll
    for (int m = 0; m < M; ++m) tot[m] = 0.0f;

    for (int gb = wave; gb < ng; gb += kGemvWaves * kGemvBatch) {
        uint4 cw[kGemvBatch];
        float sc[kGemvBatch];
#pragma unroll
        for (int u = 0; u < kGemvBatch; ++u) {
            const int gl = gb + u * kGemvWaves;
            if (gl < ng) {
                cw[u] = *reinterpret_cast<const uint4*>(cbase + int64_t(gl) * kChunkBytes);
                sc[u] = sbase[int64_t(gl) * kTileRows];
            } else {
                cw[u] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
                sc[u] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kGemvBatch; ++u) {
            const int gl = gb + u * kGemvWaves;
            if (gl >= ng) break;
            const uint32_t words[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint16_t* xp = xs + m * klen + gl * kGroup + 8 * kq;
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 xv = *reinterpret_cast<const uint4*>(xp + 32 * s);
                    acc = dot2<ACT>(magic_pair<ACT>(words[s], 0), xv.x, acc);
                    acc = dot2<ACT>(magic_pair<ACT>(words[s], 1), xv.y, acc);
                    acc = dot2<ACT>(magic_pair<ACT>(words[s], 2), xv.z, acc);
                    acc = dot2<ACT>(magic_pair<ACT>(words[s], 3), xv.w, acc);
                }
                acc = fmaf(-off, xsum[(m * ng + gl) * 4 + kq], acc);
                tot[m] = fmaf(sc[u], acc, tot[m]);
            }
        }
    }

    // Rows: sum the 4 lane-quarters, then the 4 waves.
#pragma unroll
    for (int m = 0; m < M; ++m) {
        tot[m] += __shfl_xor(tot[m], 16);
        tot[m] += __shfl_xor(tot[m], 32);
        if (lane < 16) red[(wave * M + m) * 16 + lane] = tot[m];
    }
    __syncthreads();

    float v = 0.0f;
    const int om = tid >> 4, orow = tid & 15;
    const bool owner = tid < M * 16;
    if (owner) {
#pragma unroll
        for (int w = 0; w < kGemvWaves; ++w) v += red[(w * M + om) * 16 + orow];
    }

    if (a.splits > 1) {
        __shared__ int last;
        if (owner) a.partials[((tl * a.splits + split) * M + om) * 16 + orow] = v;
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(a.counters + tl, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            last = prev == uint32_t(a.splits - 1);
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
        if (owner) {
            v = 0.0f;
            for (int sp = 0; sp < a.splits; ++sp)
                v += __hip_atomic_load(a.partials + ((tl * a.splits + sp) * M + om) * 16 + orow,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) __hip_atomic_store(a.counters + tl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (owner) {
        const int64_t ncol = t * kTileRows + orow;
        if (ncol < a.n) {
            if (a.bias) v += to_f32<ACT>(a.bias[ncol]);
            a.y[om * a.ldy + ncol] = from_f32<ACT>(v);
        }
    }
}

// --- planning ---------------------------------------------------------------

GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k) {
    GemvPlan p{};
    const Layout L(n, k);
    // Aim for ~1024 workgroups (4 per CU on 256 CUs) with at least 4 groups
    // (one chunk per wave) and at most 32 groups (32 KB of x at M = 4) each.
    int64_t gps = ceil_div(L.chunks(), 1024);
    gps = gps < 4 ? 4 : gps;
    gps = gps > 32 ? 32 : gps;
    gps = gps > L.groups ? L.groups : gps;
    p.gps = int(gps);
    p.splits = int(ceil_div(L.groups, gps));
    p.tiles_per_launch = p.splits > 1 && L.tiles > kMaxSlots ? kMaxSlots : L.tiles;
    const int mm = int(m);
    p.lds = size_t(mm) * gps * kGroup * 2 + size_t(mm) * gps * 4 * 4 + size_t(kGemvWaves) * mm * 16 * 4;
    p.workspace = p.splits > 1 ? workspace_layout_bytes(size_t(p.tiles_per_launch) * p.splits * mm * 16) : 0;
    return p;
}

template <int M, int ACT>
static void launch_one(GemvArgs a, const GemvPlan& p, hipStream_t stream) {
    const Layout L(a.n, a.k);
    for (int64_t t0 = 0; t0 < L.tiles; t0 += p.tiles_per_launch) {
        const int64_t nt = L.tiles - t0 < p.tiles_per_launch ? L.tiles - t0 : p.tiles_per_launch;
        a.t0 = t0;
        gemv_kernel<M, ACT><<<dim3(unsigned(nt * p.splits)), dim3(kGemvThreads), p.lds, stream>>>(a);
    }
}

hipError_t launch_gemv(const void* x, int act, int64_t m, int64_t k, int64_t ldx, const void* packed,
                       int64_t n, const void* bias, void* y, int64_t ldy, void* workspace,
                       hipStream_t stream) {
    const GemvPlan p = plan_gemv(m, n, k);
    GemvArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.ldx = ldx;
    a.packed = static_cast<const uint8_t*>(packed);
    a.n = n;
    a.k = k;
    a.bias = static_cast<const uint16_t*>(bias);
    a.y = static_cast<uint16_t*>(y);
    a.ldy = ldy;
    a.counters = static_cast<uint32_t*>(workspace);
    a.partials = workspace ? workspace_partials(workspace) : nullptr;
    a.t0 = 0;
    a.splits = p.splits;
    a.gps = p.gps;
    const bool bf = act == kActBf16;
    switch (m) {
        case 1: bf ? launch_one<1, kActBf16>(a, p, stream) : launch_one<1, kActF16>(a, p, stream); break;
        case 2: bf ? launch_one<2, kActBf16>(a, p, stream) : launch_one<2, kActF16>(a, p, stream); break;
        case 3: bf ? launch_one<3, kActBf16>(a, p, stream) : launch_one<3, kActF16>(a, p, stream); break;
        default: bf ? launch_one<4, kActBf16>(a, p, stream) : launch_one<4, kActF16>(a, p, stream); break;
    }
    return hipGetLastError();
}

}  // namespace w4a16
