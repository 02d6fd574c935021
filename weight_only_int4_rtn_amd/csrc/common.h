// Shared definitions of the HIP library: the packed weight layout, 16-bit
// conversions and launch planning.  gfx950 (CDNA4) only: wave64, MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace w4a16 {

// ---------------------------------------------------------------------------
// Packed execution layout ("the physical form" of a quantized weight).
//
// The [N][K] weight is cut into chunks of 16 rows x 128 columns (one scale
// group per row).  T = ceil(N/16) row tiles, G = K/128 groups.
//
//   codes region : T*G chunks of 1024 bytes, chunk (t, g) at (t*G + g)*1024.
//   scale region : after the codes, 16 FP32 per chunk, chunk (t, g) at
//                  T*G*1024 + (t*G + g)*64, entry r = row 16t + r.
//
// Inside a chunk, lane L of a wave (0..63) owns bytes [16L, 16L + 16): four
// 32-bit words w[s], s = 0..3.  Lane L stands for row r = L % 16 and quarter
// kq = L / 16; word s holds the 8 codes of columns
//     k = 128g + 32s + 8kq + j,   j = 0..7,
// as offset-binary nibbles u = q + 8: nibble i (bits 4i..4i+3, i = 0..3)
// holds column j = 2i and nibble i + 4 holds column j = 2i + 1.  So
//     ((w >> 4i) & 0x000F000F)
// puts columns (2i, 2i+1) into the low and high 16-bit halves, ready to be
// turned into a packed pair of 16-bit floats.  This is also exactly the
// B-operand layout of v_mfma_f32_16x16x32_{bf16,f16} for k-step s (lane L:
// column n = L % 16, k = 8*(L/16) + j).  Rows n >= N of the last tile hold
// code 0 (u = 8) and scale 0.
//
// INT8 weights use the same tiles, chunks and scale region with 2048-byte
// chunks of one byte per code, u = q + 128.  A chunk is two 1 KB halves:
// half h holds k-steps 2h and 2h + 1, and lane L owns bytes
// [1024h + 16L, 1024h + 16L + 16) of it, four words w[j] = the 4 codes of
// columns
//     k = 128g + 32(2h + j/2) + 8kq + 4(j%2) + b,   byte b = 0..3,
// so a wave reads each half with one contiguous 1 KB load and words 2j', 2j'+1
// of a half form the same MFMA B operand (k-step, lane) as above.  Rows
// n >= N of the last tile hold code 0 (u = 128) and scale 0.
// ---------------------------------------------------------------------------
constexpr int kGroup = 128;
constexpr int kTileRows = 16;
constexpr int kChunkBytes = 1024;
constexpr int kChunkBytes8 = 2048;
constexpr int kChunkScaleBytes = 64;

template <int BITS>
__host__ __device__ inline constexpr int chunk_bytes() { return BITS == 8 ? kChunkBytes8 : kChunkBytes; }

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Layout {
    int64_t n, k, tiles, groups, cb;  // cb: code bytes of one chunk
    __host__ __device__ Layout(int64_t n_, int64_t k_, int bits = 4)
        : n(n_), k(k_), tiles(ceil_div(n_, kTileRows)), groups(k_ / kGroup),
          cb(bits == 8 ? kChunkBytes8 : kChunkBytes) {}
    __host__ __device__ int64_t chunks() const { return tiles * groups; }
    __host__ __device__ int64_t scale_offset() const { return chunks() * cb; }
    __host__ __device__ int64_t bytes() const { return chunks() * (cb + kChunkScaleBytes); }
};

// Offset-binary nibble value of the packed-pair magic numbers.
//  bf16 0x4300 = 128.0 (spacing 1), so 0x4300 | u = 128 + u = 136 + q.
//  f16  0x6400 = 1024.0 (spacing 1), so 0x6400 | u = 1024 + u = 1032 + q.
constexpr uint32_t kMagicBf16x2 = 0x43004300u;
constexpr uint32_t kMagicF16x2 = 0x64006400u;
constexpr float kOffsetBf16 = 136.0f;
constexpr float kOffsetF16 = 1032.0f;

enum ActType { kActBf16 = 1, kActF16 = 2 };

// ---------------------------------------------------------------------------
// 16-bit float helpers (device).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int ACT>
__device__ inline float to_f32(uint16_t bits) {
    if constexpr (ACT == kActBf16) {
        return __uint_as_float(uint32_t(bits) << 16);
    } else {
        return float(__builtin_bit_cast(_Float16, bits));
    }
}

// Round-to-nearest-even conversion of an FP32 value to the activation dtype.
template <int ACT>
__device__ inline uint16_t from_f32(float v) {
    if constexpr (ACT == kActBf16) {
        return __builtin_bit_cast(uint16_t, (__bf16)v);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    }
}

// Dot product of two packed pairs accumulated in FP32:
// acc + a.lo*b.lo + a.hi*b.hi (v_dot2_f32_bf16 / v_dot2_f32_f16).
template <int ACT>
__device__ inline float dot2(uint32_t a, uint32_t b, float acc) {
    if constexpr (ACT == kActBf16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), acc, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), acc, false);
    }
}

// Sum of the eight 16-bit values of a 16-byte x load in FP32: four v_dot2
// against (1, 1) (exact products, FP32 accumulation) instead of eight
// conversions and seven additions.
template <int ACT>
__device__ inline float sum8(uint4 v) {
    constexpr uint32_t ones = ACT == kActBf16 ? 0x3F803F80u : 0x3C003C00u;
    float s = dot2<ACT>(v.x, ones, 0.0f);
    s = dot2<ACT>(v.y, ones, s);
    s = dot2<ACT>(v.z, ones, s);
    return dot2<ACT>(v.w, ones, s);
}

// i / d for 0 <= i < 2^13 and d >= 1 without an integer division sequence
// (inv_d = 1.0f / d): (i + 1/2) / d lies at least 1/(2d) from an integer,
// and its FP32 evaluation errs by less than (i + 1/2) / d * 2^-23 < 2^-10 / d,
// so the truncation is exact.
__device__ inline int div_small(int i, float inv_d) { return int((float(i) + 0.5f) * inv_d); }

// (a & mask) | bits in one v_and_or_b32.  gfx9 VOP3 encodings take no
// literal constants, so the compiler would otherwise emit a separate and + or
// pair; the operands here are registers (constants hoisted out of loops).
__device__ inline uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(mask), "v"(bits));
    return d;
}

// Packed pair (columns 2i, 2i+1 of a word) as two 16-bit floats off + q.
template <int ACT>
__device__ inline uint32_t magic_pair(uint32_t word, int i) {
    constexpr uint32_t magic = ACT == kActBf16 ? kMagicBf16x2 : kMagicF16x2;
    return and_or(i == 0 ? word : word >> (4 * i), 0x000F000Fu, magic);
}

// ---------------------------------------------------------------------------
// Activations fused into a layer's input ("Piper Kernels", section "ConvRot
// INT8"): SwiGLU rows hold [up | gate] (2K values) and give up * silu(gate);
// GELU rows give the tanh-approximate GELU.  Evaluated in FP32 and rounded
// once to the activation dtype (nearest even).  (1 + tanh u) / 2 is written
// as 1 / (1 + e^-2u): the same function without the cancellation of
// 1 + tanh(u) for large negative inputs.
// ---------------------------------------------------------------------------
enum ActFn { kActFnNone = 0, kActFnSwiglu = 1, kActFnGeluTanh = 2 };

// The logistic factor takes the hardware reciprocal (v_rcp_f32, about one
// FP32 ulp) rather than a correctly rounded division: the result is rounded
// to 16 bits next, and every workgroup recomputes the activation of its slice.
__device__ inline float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ inline float gelu_tanh_f32(float x) {
    const float u = 0.7978845608028654f * fmaf(0.044715f * x, x * x, x);  // sqrt(2/pi) (x + 0.044715 x^3)
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * u));
}

// Eight 16-bit inputs (and, for SwiGLU, the eight matching gate values) ->
// eight activated 16-bit values, in place order.
template <int ACT, int AF>
__device__ inline uint4 activate8(uint4 v, uint4 g) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w}, gt[4] = {g.x, g.y, g.z, g.w};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo = to_f32<ACT>(uint16_t(in[i] & 0xFFFFu)), hi = to_f32<ACT>(uint16_t(in[i] >> 16));
        if constexpr (AF == kActFnSwiglu) {
            lo *= silu_f32(to_f32<ACT>(uint16_t(gt[i] & 0xFFFFu)));
            hi *= silu_f32(to_f32<ACT>(uint16_t(gt[i] >> 16)));
        } else {
            lo = gelu_tanh_f32(lo);
            hi = gelu_tanh_f32(hi);
        }
        out[i] = uint32_t(from_f32<ACT>(lo)) | (uint32_t(from_f32<ACT>(hi)) << 16);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// 16-byte load of streamed data (read once: nontemporal, so it does not
// displace data the kernel reuses from the caches).
__device__ inline uint4 load_stream16(const uint8_t* p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A value the same in every lane, kept in a scalar register (buffer
// resources and offsets must be; per-wave indices computed from it stay on
// the scalar unit instead of costing vector instructions in every lane).
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Buffer resource over `bytes` bytes from `base` (bytes < 2^31); loads past
// the end return zero.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = uint32_t(uniform(int(uint32_t(b)))), hi = uint32_t(uniform(int(uint32_t(b >> 32))));
    void* p = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, uniform(int(uint32_t(bytes))), 0x00020000);
}

// Cache-policy operand of a buffer load: nontemporal (data read once).
constexpr int kBufNontemporal = 2;
// Cache-policy operand of a buffer access at device scope (SC1): stores write
// through the L2 and loads read past it, so workgroups on different XCDs
// see each other's data without L2 write-backs or invalidations.
constexpr int kCoherent = 16;

// v of lane (lane ^ M), M a power of two below 32: one ds_swizzle in bitmask
// mode (__shfl_xor spends several vector instructions per call on the lane
// index and its bounds).
template <int M>
__device__ inline float lane_xor(float v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16, "swizzle mask");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

// v(lane) + v(lane ^ 32), and the same with max: one v_permlane32_swap gives
// each lane the pair {v(lane), v(lane ^ 32)} (in either order; both
// operations are commutative, so every lane gets the same bits).
__device__ inline float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// f(std::integral_constant<int, I>) for I = B .. E - 1 in order (a loop whose
// index is a constant expression in the body).
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// LDS address operand of the direct global-to-LDS buffer loads.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Waits until at most N vector memory operations of this wave are in flight
// (they complete in issue order).  For loads the compiler cannot track, such
// as direct global-to-LDS loads, which write no register.  s_waitcnt's
// immediate on gfx9: vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8
// (those two left at their maxima: no wait).
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, then s_barrier.  __syncthreads() also waits for every
// outstanding global load (vmcnt(0)), which would serialise the weight
// prefetch that is in flight when x is staged.
__device__ inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Packed pair of the two codes in bytes (2h, 2h + 1) of an INT8 word (h = 0,
// 1) as two 16-bit floats holding off + q exactly:
//  f16: 0x6400 | u = 1024 + u = 1152 + q (one v_perm placing the bytes, one or);
//  bf16: u itself (8 significant bits fit bf16's 8): each byte converted to
//        FP32 (v_cvt_f32_ubyte), whose upper halves are the exact bf16 values.
template <int ACT>
__device__ inline uint32_t byte_pair(uint32_t word, int h) {
    if constexpr (ACT == kActF16) {
        return __builtin_amdgcn_perm(0u, word, h == 0 ? 0x0c010c00u : 0x0c030c02u) | kMagicF16x2;
    } else {
        const float lo = float((word >> (16 * h)) & 0xFFu);
        const float hi = float((word >> (16 * h + 8)) & 0xFFu);
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
}

// The four packed pairs (columns 8kq + 0..7 of k-step s) of a lane's chunk
// data: w holds the lane's 4 words (INT4) or 8 words (INT8, both halves).
template <int BITS, int ACT>
__device__ inline uint4 bpairs(const uint32_t* w, int s) {
    if constexpr (BITS == 8) {
        const uint32_t a = w[2 * s], b = w[2 * s + 1];
        return make_uint4(byte_pair<ACT>(a, 0), byte_pair<ACT>(a, 1), byte_pair<ACT>(b, 0), byte_pair<ACT>(b, 1));
    } else {
        return make_uint4(magic_pair<ACT>(w[s], 0), magic_pair<ACT>(w[s], 1), magic_pair<ACT>(w[s], 2),
                          magic_pair<ACT>(w[s], 3));
    }
}

// v >> N as one v_lshrrev_b64 (the compiler would split it into a funnel
// shift and a 32-bit shift).
template <int N>
__device__ inline uint64_t shr64(uint64_t v) {
    uint64_t d;
    asm("v_lshrrev_b64 %0, %1, %2" : "=v"(d) : "i"(N), "v"(v));
    return d;
}

// The packed pairs of k-steps s and s + 1 (s even) of a lane's chunk data,
// b[h] = bpairs(w, s + h).  INT4 words go two at a time through 64-bit
// shifts: one shift serves both words (the bits it carries from the upper
// word into the lower fall outside the 0x000F000F mask), 1.5 shifts per word
// instead of 3.
template <int BITS, int ACT>
__device__ inline void bpairs2(const uint32_t* w, int s, uint4 (&b)[2]) {
    if constexpr (BITS == 8) {
        b[0] = bpairs<BITS, ACT>(w, s);
        b[1] = bpairs<BITS, ACT>(w, s + 1);
    } else {
        constexpr uint32_t magic = ACT == kActBf16 ? kMagicBf16x2 : kMagicF16x2;
        const uint64_t v = uint64_t(w[s]) | (uint64_t(w[s + 1]) << 32);
        const uint64_t sh[4] = {v, shr64<4>(v), shr64<8>(v), shr64<12>(v)};
#pragma unroll
        for (int h = 0; h < 2; ++h)
            b[h] = make_uint4(and_or(uint32_t(sh[0] >> (32 * h)), 0x000F000Fu, magic),
                              and_or(uint32_t(sh[1] >> (32 * h)), 0x000F000Fu, magic),
                              and_or(uint32_t(sh[2] >> (32 * h)), 0x000F000Fu, magic),
                              and_or(uint32_t(sh[3] >> (32 * h)), 0x000F000Fu, magic));
    }
}

// The offset each packed pair value carries: off + q.
template <int ACT, int BITS = 4>
__device__ inline constexpr float code_offset() {
    if constexpr (BITS == 8) return ACT == kActBf16 ? 128.0f : 1152.0f;
    return ACT == kActBf16 ? kOffsetBf16 : kOffsetF16;
}

}  // namespace w4a16
