// Load-time kernels: round-to-nearest INT4 quantization with one FP32 scale
// per group of 128 ("Kernel dispatch and Humming quantization in PhyAI",
// section "Humming makes the separation useful"), and the lowering of the
// canonical codes and scales into the packed execution layout (common.h).
//
// These run once per weight; they are HBM-bound streaming kernels.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

// ---------------------------------------------------------------------------
// Quantization.  One thread owns 8 consecutive weights of a row; the 16
// threads of a group (adjacent lanes, since k/8 is a multiple of 16) reduce
// their largest magnitude with cross-lane exchanges.
//
//   s = amax / 7           correctly rounded FP32 division (no reciprocal)
//   q = clamp(rint(w / s), -8, 7), q = 0 when s == 0
// rint is v_rndne_f32: round half to even.  Denormals are kept (the library
// is compiled without flush-to-zero), so tiny groups round exactly like the
// IEEE definition.
// ---------------------------------------------------------------------------
template <int DT>  // 0 = f32, 1 = bf16, 2 = f16 (w4a16_dtype_t numbering)
__device__ inline void load_weights8(const void* base, int64_t idx, float v[8]) {
    if constexpr (DT == 0) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
        uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t lo = uint16_t(w[i] & 0xFFFFu), hi = uint16_t(w[i] >> 16);
            v[2 * i] = DT == 1 ? to_f32<kActBf16>(lo) : to_f32<kActF16>(lo);
            v[2 * i + 1] = DT == 1 ? to_f32<kActBf16>(hi) : to_f32<kActF16>(hi);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ w, int64_t n,
                                                       int64_t k, int64_t ldw,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
    const int64_t per_row = k / 8;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = n * per_row;
    // Every thread of a 16-lane group is either in range or not: total is a
    // multiple of 16 and 16-lane groups never straddle the end.
    const bool active = tid < total;
    const int64_t row = active ? tid / per_row : 0;
    const int64_t k0 = active ? (tid - row * per_row) * 8 : 0;

    float v[8];
    if (active) {
        load_weights8<DT>(w, row * ldw + k0, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // reduce over the 16 threads of the group (lanes differing in bits 0..3)
    amax = fmaxf(amax, lane_xor<1>(amax));
    amax = fmaxf(amax, lane_xor<2>(amax));
    amax = fmaxf(amax, lane_xor<4>(amax));
    amax = fmaxf(amax, lane_xor<8>(amax));
    if (!active) return;

    const float s = amax / 7.0f;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s != 0.0f) {
            float r = rintf(v[i] / s);
            r = fminf(fmaxf(r, -8.0f), 7.0f);
            q = int(r);
        }
        word |= (uint32_t(q) & 0xFu) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(codes + row * (k / 2) + k0 / 2) = word;
    if ((k0 & (kGroup - 1)) == 0) scales[row * (k / kGroup) + k0 / kGroup] = s;
}

hipError_t launch_quantize(const void* w, int dtype, int64_t n, int64_t k, int64_t ldw,
                           uint8_t* codes, float* scales, hipStream_t stream) {
    const int64_t total = n * (k / 8);
    const int64_t blocks = ceil_div(total, 256);
    switch (dtype) {
        case 0: quantize_kernel<0><<<dim3(blocks), dim3(256), 0, stream>>>(w, n, k, ldw, codes, scales); break;
        case 1: quantize_kernel<1><<<dim3(blocks), dim3(256), 0, stream>>>(w, n, k, ldw, codes, scales); break;
        default: quantize_kernel<2><<<dim3(blocks), dim3(256), 0, stream>>>(w, n, k, ldw, codes, scales); break;
    }
    return hipGetLastError();
}

// INT8 (the same method with the 8-bit code range): s = amax / 127,
// q = clamp(rint(w / s), -128, 127), q = 0 when s == 0; one signed code per
// byte, 8 bytes per thread.
template <int DT>
__global__ __launch_bounds__(256) void quantize8_kernel(const void* __restrict__ w, int64_t n, int64_t k,
                                                        int64_t ldw, int8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
    const int64_t per_row = k / 8;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = n * per_row;
    const bool active = tid < total;  // whole 16-lane groups, as above
    const int64_t row = active ? tid / per_row : 0;
    const int64_t k0 = active ? (tid - row * per_row) * 8 : 0;

    float v[8];
    if (active) {
        load_weights8<DT>(w, row * ldw + k0, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, lane_xor<1>(amax));
    amax = fmaxf(amax, lane_xor<2>(amax));
    amax = fmaxf(amax, lane_xor<4>(amax));
    amax = fmaxf(amax, lane_xor<8>(amax));
    if (!active) return;

    const float s = amax / 127.0f;
    uint32_t word[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s != 0.0f) q = int(fminf(fmaxf(rintf(v[i] / s), -128.0f), 127.0f));
        word[i >> 2] |= (uint32_t(q) & 0xFFu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(codes + row * k + k0) = make_uint2(word[0], word[1]);
    if ((k0 & (kGroup - 1)) == 0) scales[row * (k / kGroup) + k0 / kGroup] = s;
}

hipError_t launch_quantize8(const void* w, int dtype, int64_t n, int64_t k, int64_t ldw, int8_t* codes,
                            float* scales, hipStream_t stream) {
    const int64_t blocks = ceil_div(n * (k / 8), 256);
    switch (dtype) {
        case 0: quantize8_kernel<0><<<dim3(blocks), dim3(256), 0, stream>>>(w, n, k, ldw, codes, scales); break;
        case 1: quantize8_kernel<1><<<dim3(blocks), dim3(256), 0, stream>>>(w, n, k, ldw, codes, scales); break;
        default: quantize8_kernel<2><<<dim3(blocks), dim3(256), 0, stream>>>(w, n, k, ldw, codes, scales); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Canonical <-> packed.  One thread per (chunk, lane): four words.
// Canonical word for 8 consecutive columns k0..k0+7 of a row: byte b holds
// column k0+2b in the low nibble and k0+2b+1 in the high nibble (two's
// complement).  Packed word: nibble i = u(k0+2i), nibble i+4 = u(k0+2i+1),
// u = q + 8 = c ^ 8 for a two's-complement nibble c.
// ---------------------------------------------------------------------------
__device__ inline uint32_t canonical_to_packed(uint32_t c) {
    uint32_t p = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t lo = ((c >> (8 * b)) & 0xFu) ^ 0x8u;
        uint32_t hi = ((c >> (8 * b + 4)) & 0xFu) ^ 0x8u;
        p |= lo << (4 * b);
        p |= hi << (4 * b + 16);
    }
    return p;
}

__device__ inline uint32_t packed_to_canonical(uint32_t p) {
    uint32_t c = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t lo = ((p >> (4 * b)) & 0xFu) ^ 0x8u;
        uint32_t hi = ((p >> (4 * b + 16)) & 0xFu) ^ 0x8u;
        c |= (lo | (hi << 4)) << (8 * b);
    }
    return c;
}

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   const float* __restrict__ scales, int64_t n,
                                                   int64_t k, uint8_t* __restrict__ packed) {
    const Layout L(n, k);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (tid >= L.chunks() * 64) return;
    const int64_t chunk = tid >> 6;
    const int lane = int(tid & 63);
    const int64_t t = chunk / L.groups, g = chunk - t * L.groups;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t row = t * kTileRows + r;
    uint32_t out[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int64_t k0 = g * kGroup + 32 * s + 8 * kq;
        out[s] = row < n ? canonical_to_packed(*reinterpret_cast<const uint32_t*>(codes + row * (k / 2) + k0 / 2))
                         : 0x88888888u;
    }
    *reinterpret_cast<uint4*>(packed + chunk * kChunkBytes + lane * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    if (kq == 0) {
        float* sp = reinterpret_cast<float*>(packed + L.scale_offset());
        sp[chunk * kTileRows + r] = row < n ? scales[row * L.groups + g] : 0.0f;
    }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed, int64_t n,
                                                     int64_t k, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales) {
    const Layout L(n, k);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (tid >= L.chunks() * 64) return;
    const int64_t chunk = tid >> 6;
    const int lane = int(tid & 63);
    const int64_t t = chunk / L.groups, g = chunk - t * L.groups;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t row = t * kTileRows + r;
    if (row >= n) return;
    uint4 in = *reinterpret_cast<const uint4*>(packed + chunk * kChunkBytes + lane * 16);
    uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int64_t k0 = g * kGroup + 32 * s + 8 * kq;
        *reinterpret_cast<uint32_t*>(codes + row * (k / 2) + k0 / 2) = packed_to_canonical(w[s]);
    }
    if (kq == 0) {
        const float* sp = reinterpret_cast<const float*>(packed + L.scale_offset());
        scales[row * L.groups + g] = sp[chunk * kTileRows + r];
    }
}

// INT8 canonical <-> packed.  One thread per (chunk, lane, half): four words,
// each the 4 consecutive columns 128g + 32(2h + j/2) + 8kq + 4(j%2) .. +3 of
// the lane's row; u = q + 128 is the two's-complement byte with its top bit
// flipped, so a word converts with one xor.
__global__ __launch_bounds__(256) void pack8_kernel(const int8_t* __restrict__ codes,
                                                    const float* __restrict__ scales, int64_t n, int64_t k,
                                                    uint8_t* __restrict__ packed) {
    const Layout L(n, k, 8);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (tid >= L.chunks() * 128) return;
    const int64_t chunk = tid >> 7;
    const int h = int((tid >> 6) & 1), lane = int(tid & 63);
    const int64_t t = chunk / L.groups, g = chunk - t * L.groups;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t row = t * kTileRows + r;
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t k0 = g * kGroup + 32 * (2 * h + j / 2) + 8 * kq + 4 * (j % 2);
        out[j] = row < n ? *reinterpret_cast<const uint32_t*>(codes + row * k + k0) ^ 0x80808080u : 0x80808080u;
    }
    *reinterpret_cast<uint4*>(packed + chunk * kChunkBytes8 + h * kChunkBytes + lane * 16) =
        make_uint4(out[0], out[1], out[2], out[3]);
    if (h == 0 && kq == 0) {
        float* sp = reinterpret_cast<float*>(packed + L.scale_offset());
        sp[chunk * kTileRows + r] = row < n ? scales[row * L.groups + g] : 0.0f;
    }
}

__global__ __launch_bounds__(256) void unpack8_kernel(const uint8_t* __restrict__ packed, int64_t n, int64_t k,
                                                      int8_t* __restrict__ codes, float* __restrict__ scales) {
    const Layout L(n, k, 8);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (tid >= L.chunks() * 128) return;
    const int64_t chunk = tid >> 7;
    const int h = int((tid >> 6) & 1), lane = int(tid & 63);
    const int64_t t = chunk / L.groups, g = chunk - t * L.groups;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t row = t * kTileRows + r;
    if (row >= n) return;
    const uint4 in = *reinterpret_cast<const uint4*>(packed + chunk * kChunkBytes8 + h * kChunkBytes + lane * 16);
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t k0 = g * kGroup + 32 * (2 * h + j / 2) + 8 * kq + 4 * (j % 2);
        *reinterpret_cast<uint32_t*>(codes + row * k + k0) = w[j] ^ 0x80808080u;
    }
    if (h == 0 && kq == 0) {
        const float* sp = reinterpret_cast<const float*>(packed + L.scale_offset());
        scales[row * L.groups + g] = sp[chunk * kTileRows + r];
    }
}

hipError_t launch_pack8(const int8_t* codes, const float* scales, int64_t n, int64_t k, void* packed,
                        hipStream_t stream) {
    const Layout L(n, k, 8);
    const int64_t blocks = ceil_div(L.chunks() * 128, 256);
    pack8_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(codes, scales, n, k, static_cast<uint8_t*>(packed));
    return hipGetLastError();
}

hipError_t launch_unpack8(const void* packed, int64_t n, int64_t k, int8_t* codes, float* scales,
                          hipStream_t stream) {
    const Layout L(n, k, 8);
    const int64_t blocks = ceil_div(L.chunks() * 128, 256);
    unpack8_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(static_cast<const uint8_t*>(packed), n, k, codes,
                                                           scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shard of a packed weight without requantizing ("Piper Kernels", section
// "NVFP4 construction", partitioning an already quantized weight: the packed
// data is copied, nibble order and scales preserved).  One thread per
// (output chunk, lane): 16 bytes.
//   dim 0: output rows r of [0, len) are source rows start + r (any start);
//          a row moves as the four 16-byte lane runs (one per k-quarter) of
//          each of its chunks, plus its scale.  Rows past len in the last
//          output tile get code 0 (nibble 8) and scale 0, as pack writes them.
//   dim 1: output groups are source groups start/128 + g': whole chunks and
//          their scale blocks are copied.
// ---------------------------------------------------------------------------
// BITS 8: INT8 chunks, whose lane runs sit in two 1 KB halves (each moved
// alike); padding rows get code 0 as u = 0x80.
template <int BITS>
__global__ __launch_bounds__(256) void shard_kernel(const uint8_t* __restrict__ src, int64_t n, int64_t k,
                                                    int dim, int64_t start, int64_t len,
                                                    uint8_t* __restrict__ dst) {
    constexpr int CB = chunk_bytes<BITS>(), H = BITS / 4;
    constexpr uint32_t kZero = BITS == 8 ? 0x80808080u : 0x88888888u;
    const Layout S(n, k, BITS);
    const Layout D(dim == 0 ? len : n, dim == 0 ? k : len, BITS);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (tid >= D.chunks() * 64) return;
    const int64_t chunk = tid >> 6;
    const int lane = int(tid & 63);
    const int64_t t = chunk / D.groups, g = chunk - t * D.groups;
    const int r = lane & 15, kq = lane >> 4;
    const float* ss = reinterpret_cast<const float*>(src + S.scale_offset());
    float* ds = reinterpret_cast<float*>(dst + D.scale_offset());
    uint4 v[H];
    float sc;
    if (dim == 0) {
        const int64_t orow = t * kTileRows + r;
        if (orow < len) {
            const int64_t srow = start + orow;
            const int64_t schunk = (srow / kTileRows) * S.groups + g;
            const int slane = int(srow % kTileRows) + 16 * kq;
#pragma unroll
            for (int h = 0; h < H; ++h)
                v[h] = *reinterpret_cast<const uint4*>(src + schunk * CB + h * kChunkBytes + slane * 16);
            sc = ss[schunk * kTileRows + srow % kTileRows];
        } else {
#pragma unroll
            for (int h = 0; h < H; ++h) v[h] = make_uint4(kZero, kZero, kZero, kZero);
            sc = 0.0f;
        }
    } else {
        const int64_t schunk = t * S.groups + start / kGroup + g;
#pragma unroll
        for (int h = 0; h < H; ++h)
            v[h] = *reinterpret_cast<const uint4*>(src + schunk * CB + h * kChunkBytes + lane * 16);
        sc = ss[schunk * kTileRows + r];
    }
#pragma unroll
    for (int h = 0; h < H; ++h) *reinterpret_cast<uint4*>(dst + chunk * CB + h * kChunkBytes + lane * 16) = v[h];
    if (kq == 0) ds[chunk * kTileRows + r] = sc;
}

hipError_t launch_shard(const void* packed, int64_t n, int64_t k, int dim, int64_t start, int64_t len,
                        void* out, int bits, hipStream_t stream) {
    const Layout D(dim == 0 ? len : n, dim == 0 ? k : len, bits);
    const int64_t blocks = ceil_div(D.chunks() * 64, 256);
    const uint8_t* src = static_cast<const uint8_t*>(packed);
    uint8_t* dst = static_cast<uint8_t*>(out);
    if (bits == 8)
        shard_kernel<8><<<dim3(blocks), dim3(256), 0, stream>>>(src, n, k, dim, start, len, dst);
    else
        shard_kernel<4><<<dim3(blocks), dim3(256), 0, stream>>>(src, n, k, dim, start, len, dst);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                       void* packed, hipStream_t stream) {
    const Layout L(n, k);
    const int64_t blocks = ceil_div(L.chunks() * 64, 256);
    pack_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(codes, scales, n, k, static_cast<uint8_t*>(packed));
    return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, int64_t n, int64_t k, uint8_t* codes, float* scales,
                         hipStream_t stream) {
    const Layout L(n, k);
    const int64_t blocks = ceil_div(L.chunks() * 64, 256);
    unpack_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(static_cast<const uint8_t*>(packed), n, k, codes, scales);
    return hipGetLastError();
}

}  // namespace w4a16
