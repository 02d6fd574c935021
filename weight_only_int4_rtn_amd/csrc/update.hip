// In-place update of a packed weight ("Piper Kernels", sections "ConvRot
// INT8" -- add_ / addmm_ requantize the updated weight, an optional 64-bit
// rounding_seed selects stochastic rounding without changing the scales --
// and "Stochastic quantization" -- one of the two adjacent codes with
// probability proportional to distance, values outside the code range and
// exact hits never perturbed, draws by logical element offset).
//
//   W' = beta * dequant(W) + alpha * U,  U = dense update, or mat1 @ mat2
//
// Each step is one FP32 operation: d = fl32(q * s); p = U, or the FMA chain
// p = fma(mat1[n][r], mat2[r][k], p) over r ascending; w' = fma(alpha, p,
// fl32(beta * d)).  Then the round-to-nearest quantizer (scale amax / 7 over
// the group, correctly rounded quotient) picks the scale, and each code is
// nearest (no seed) or floor(v) + (u < v - floor(v)) for interior quotients
// v, with u the top 24 bits of draw e = n * K + k of SplitMix64 (Steele, Lea
// and Flood, OOPSLA 2014) seeded with the 64-bit seed.
//
// One thread per (chunk, lane) of the packed layout: the lane's 32 weights
// (16 bytes, INT8: two 16-byte runs) of one row and group quarter.  INT8
// weights (BITS 8) take the INT8 quantizer: scale amax / 127, codes
// [-128, 127], stochastic rounding where -128 <= floor(v) <= 126.  The four lanes of a row (L,
// L+16, L+32, L+48 of the same wave) combine their magnitudes with two
// cross-lane exchanges; every lane reads its words and the row's scale
// before any lane writes (one wave), so the update is in place.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

struct UpdateArgs {
    uint8_t* packed;
    int64_t n, k;
    const void* upd;   // dense [n][ldu] or null
    int64_t ldu;
    const void* mat1;  // [n][rank]
    const void* mat2;  // [rank][k]
    int64_t rank;
    float alpha, beta;
    int stochastic;
    uint64_t seed;
};

__device__ inline uint64_t splitmix64(uint64_t seed, uint64_t e) {
    uint64_t z = seed + (e + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Element idx of an F32 / BF16 / F16 array, widened exactly to FP32.
template <int DT>
__device__ inline float elem_f32(const void* p, int64_t idx) {
    if constexpr (DT == 0) return static_cast<const float*>(p)[idx];
    else return to_f32<DT>(static_cast<const uint16_t*>(p)[idx]);
}

// Eight consecutive elements from idx (16-byte aligned for 16-bit types,
// 32-byte for FP32).
template <int DT>
__device__ inline void load8_f32(const void* p, int64_t idx, float* out) {
    if constexpr (DT == 0) {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + idx);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = to_f32<DT>(uint16_t(w[i] & 0xFFFFu));
            out[2 * i + 1] = to_f32<DT>(uint16_t(w[i] >> 16));
        }
    }
}

template <int DT, bool LOWRANK, int BITS>
__global__ __launch_bounds__(256) void update_kernel(UpdateArgs a) {
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    constexpr float kQmax = BITS == 8 ? 127.0f : 7.0f, kQmin = -kQmax - 1.0f;
    const Layout L(a.n, a.k, BITS);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t chunk = tid >> 6;
    // whole waves stay together (the grid covers whole chunks) so the row's
    // lanes exchange magnitudes; rows past n are padding and stay as they are
    if (chunk >= L.chunks()) return;
    const int lane = int(tid & 63);
    const int64_t t = chunk / L.groups, g = chunk - t * L.groups;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t row = t * kTileRows + r;
    const bool live = row < a.n;
    uint8_t* cp = a.packed + chunk * CB + lane * 16;
    float* sp = reinterpret_cast<float*>(a.packed + L.scale_offset()) + chunk * kTileRows + r;

    uint32_t words[4 * H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const uint4 in = *reinterpret_cast<const uint4*>(cp + h * kChunkBytes);
        words[4 * h] = in.x;
        words[4 * h + 1] = in.y;
        words[4 * h + 2] = in.z;
        words[4 * h + 3] = in.w;
    }
    const float s_old = *sp;

    // INT4: word s holds columns 128g + 32s + 8kq + j: nibble i = column 2i,
    // nibble i + 4 = column 2i + 1, offset-binary u = q + 8.  INT8: words
    // 2s and 2s + 1 hold columns 8kq + 0..3 and 4..7 of k-step s, one byte
    // each, u = q + 128.
    // The update U for the lane's 32 weights: dense, or the FMA chain over r
    // ascending.  The rank loop is outermost: one mat1 value per r and the
    // four k-steps' mat2 runs as independent loads (unrolled, so several
    // r are in flight); each element's chain keeps the same order.
    float pu[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) pu[i] = 0.0f;
    if (live) {
        if constexpr (LOWRANK) {
            const int64_t colg = g * kGroup + 8 * kq;
#pragma unroll 4
            for (int64_t rr = 0; rr < a.rank; ++rr) {
                const float m1 = elem_f32<DT>(a.mat1, row * a.rank + rr);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float m2[8];
                    load8_f32<DT>(a.mat2, rr * a.k + colg + 32 * s, m2);
#pragma unroll
                    for (int j = 0; j < 8; ++j) pu[8 * s + j] = fmaf(m1, m2[j], pu[8 * s + j]);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) load8_f32<DT>(a.upd, row * a.ldu + g * kGroup + 32 * s + 8 * kq, pu + 8 * s);
        }
    }
    float w[32];
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float* p = pu + 8 * s;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int qc;
            if constexpr (BITS == 8) {
                qc = int((words[2 * s + j / 4] >> (8 * (j % 4))) & 0xFFu) - 128;
            } else {
                qc = int((words[s] >> (j % 2 == 0 ? 2 * j : 16 + 2 * (j - 1))) & 0xFu) - 8;
            }
            const float d = float(qc) * s_old;
            const float bd = a.beta * d;
            const float v = fmaf(a.alpha, p[j], bd);
            w[8 * s + j] = v;
            amax = fmaxf(amax, fabsf(v));
        }
    }
    amax = fmaxf(amax, lane_xor<16>(amax));
    amax = max_xor32(amax);
    const float scale = amax / kQmax;

    uint32_t out[4 * H];
#pragma unroll
    for (int i = 0; i < 4 * H; ++i) out[i] = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int code = 0;
            if (scale != 0.0f) {
                const float v = w[8 * s + j] / scale;
                const float lo = floorf(v);
                if (a.stochastic && lo >= kQmin && lo + 1.0f <= kQmax) {
                    const int64_t col = g * kGroup + 32 * s + 8 * kq + j;
                    const uint64_t e = uint64_t(row * a.k + col);
                    const float u = float(splitmix64(a.seed, e) >> 40) * 0x1p-24f;
                    code = int(lo) + (u < v - lo ? 1 : 0);
                } else {
                    code = int(fminf(fmaxf(__builtin_rintf(v), kQmin), kQmax));
                }
            }
            if constexpr (BITS == 8) {
                out[2 * s + j / 4] |= (uint32_t(code + 128) & 0xFFu) << (8 * (j % 4));
            } else {
                out[s] |= (uint32_t(code + 8) & 0xFu) << (j % 2 == 0 ? 2 * j : 16 + 2 * (j - 1));
            }
        }
    }
    if (!live) return;
#pragma unroll
    for (int h = 0; h < H; ++h)
        *reinterpret_cast<uint4*>(cp + h * kChunkBytes) =
            make_uint4(out[4 * h], out[4 * h + 1], out[4 * h + 2], out[4 * h + 3]);
    if (kq == 0) *sp = scale;
}

template <int BITS>
static void launch_update_bits(const UpdateArgs& a, int dtype, dim3 grid, dim3 block, hipStream_t stream) {
    const bool lr = a.rank > 0;
    switch (dtype) {
        case 0:
            if (lr) update_kernel<0, true, BITS><<<grid, block, 0, stream>>>(a);
            else update_kernel<0, false, BITS><<<grid, block, 0, stream>>>(a);
            break;
        case kActBf16:
            if (lr) update_kernel<kActBf16, true, BITS><<<grid, block, 0, stream>>>(a);
            else update_kernel<kActBf16, false, BITS><<<grid, block, 0, stream>>>(a);
            break;
        default:
            if (lr) update_kernel<kActF16, true, BITS><<<grid, block, 0, stream>>>(a);
            else update_kernel<kActF16, false, BITS><<<grid, block, 0, stream>>>(a);
            break;
    }
}

hipError_t launch_update(void* packed, int64_t n, int64_t k, const void* upd, int64_t ldu, const void* mat1,
                         const void* mat2, int64_t rank, int dtype, float alpha, float beta, int stochastic,
                         uint64_t seed, int bits, hipStream_t stream) {
    const Layout L(n, k, bits);
    UpdateArgs a;
    a.packed = static_cast<uint8_t*>(packed);
    a.n = n;
    a.k = k;
    a.upd = upd;
    a.ldu = ldu;
    a.mat1 = mat1;
    a.mat2 = mat2;
    a.rank = rank;
    a.alpha = alpha;
    a.beta = beta;
    a.stochastic = stochastic;
    a.seed = seed;
    const dim3 grid(unsigned(ceil_div(L.chunks() * 64, 256))), block(256);
    if (bits == 8) launch_update_bits<8>(a, dtype, grid, block, stream);
    else launch_update_bits<4>(a, dtype, grid, block, stream);
    return hipGetLastError();
}

}  // namespace w4a16
