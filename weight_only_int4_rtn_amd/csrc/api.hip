// C ABI of the library (include/w4a16.h): argument checks from host metadata
// only, kernel choice, launches.  Nothing here allocates, synchronizes or
// reads device memory ("Piper Kernels", section "Validation contract").
#include "w4a16.h"

#include "common.h"
#include "kernels.h"

using namespace w4a16;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [lo, hi) byte ranges overlap?
bool overlap(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bn && b0 < a0 + an;
}

size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t elem) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t(rows - 1) * size_t(ld) + size_t(cols)) * elem;
}

// Sizes are limited so every internal offset fits comfortably in int64 and
// grid dimensions stay within HIP's limits.
constexpr int64_t kMaxDim = int64_t(1) << 24;
// The GEMM path addresses a 256-row x tile through one buffer resource
// (32-bit byte offsets): row stride at most 2^22 elements.
constexpr int64_t kGemmMaxLd = int64_t(1) << 22;
// Largest rank of a low-rank update (mat1 [n][rank] @ mat2 [rank][k]).
constexpr int64_t kMaxRank = int64_t(1) << 16;

bool valid_path(w4a16_path_t p) {
    return p == W4A16_PATH_AUTO || p == W4A16_PATH_GEMV || p == W4A16_PATH_MGEMV || p == W4A16_PATH_SKINNY ||
           p == W4A16_PATH_GEMM || p == W4A16_PATH_GEMM_STREAMK;
}

// the large-M kernel, with the planner's decomposition or forced stream-K
bool is_gemm(w4a16_path_t p) { return p == W4A16_PATH_GEMM || p == W4A16_PATH_GEMM_STREAMK; }

bool valid_nk(int64_t n, int64_t k) {
    return n >= 0 && n <= kMaxDim && k > 0 && k <= kMaxDim && k % kGroup == 0;
}

w4a16_status_t from_hip(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_EHIP; }

size_t path_workspace(w4a16_path_t path, int64_t m, int64_t n, int64_t k, int bits) {
    switch (path) {
        case W4A16_PATH_GEMV: {
            // row blocks of 4 and a last block of m % 4 rows, each with its own plan
            const size_t full = plan_gemv(m < 4 ? m : 4, n, k, bits).workspace;
            const size_t last = m > 4 && m % 4 ? plan_gemv(m % 4, n, k, bits).workspace : 0;
            return full > last ? full : last;
        }
        case W4A16_PATH_MGEMV: {
            // row blocks of 16 and a last block of m % 16 rows, with or
            // without a fused activation (staged or direct x operands): each
            // plan has room
            size_t most = 0;
            const int64_t blocks[2] = {m < 16 ? m : 16, m > 16 ? m % 16 : 0};
            for (const int64_t mm : blocks) {
                if (mm == 0) continue;
                for (const int fn : {int(kActFnNone), int(kActFnSwiglu)}) {
                    const size_t w = plan_mgemv(mm, n, k, bits, fn).workspace;
                    most = w > most ? w : most;
                }
            }
            return most;
        }
        case W4A16_PATH_SKINNY: {
            // the plans with and without a fused activation (different
            // workgroup widths): room for either
            const size_t direct = plan_skinny(m, n, k, bits, kActFnNone).workspace;
            const size_t staged = plan_skinny(m, n, k, bits, kActFnSwiglu).workspace;
            return direct > staged ? direct : staged;
        }
        case W4A16_PATH_GEMM: return plan_gemm(m, n, k, bits).workspace;
        case W4A16_PATH_GEMM_STREAMK: return plan_gemm_streamk(m, n, k, bits).workspace;
        default: return 0;
    }
}

// Shared argument checks of quantize (either code width).
w4a16_status_t check_quantize(const void* w, w4a16_dtype_t w_dtype, int64_t n, int64_t k, int64_t ldw,
                              const void* codes, size_t cbytes, uintptr_t calign, const float* scales) {
    if (w_dtype != W4A16_F32 && w_dtype != W4A16_BF16 && w_dtype != W4A16_F16) return W4A16_EUNSUPPORTED;
    if (!valid_nk(n, k) || ldw < k || ldw > kMaxDim) return W4A16_EINVAL;
    if (n == 0) return W4A16_OK;
    const size_t elem = w_dtype == W4A16_F32 ? 4 : 2;
    if (!w || !codes || !scales) return W4A16_EINVAL;
    if (!aligned(w, 16) || (size_t(ldw) * elem) % 16 != 0) return W4A16_EINVAL;
    if (!aligned(codes, calign) || !aligned(scales, 4)) return W4A16_EINVAL;
    const size_t wbytes = span_bytes(n, k, ldw, elem), sbytes = size_t(n) * size_t(k / kGroup) * 4;
    if (overlap(w, wbytes, codes, cbytes) || overlap(w, wbytes, scales, sbytes) ||
        overlap(codes, cbytes, scales, sbytes))
        return W4A16_EINVAL;
    return W4A16_OK;
}

// Shared argument checks of pack / unpack (either code width).
w4a16_status_t check_pack(const void* codes, size_t cbytes, const float* scales, int64_t n, int64_t k,
                          const void* packed, size_t pbytes, bool codes_out) {
    if (!valid_nk(n, k)) return W4A16_EINVAL;
    if (n == 0) return W4A16_OK;
    if (!codes || !scales || !packed) return W4A16_EINVAL;
    if (!aligned(codes, 4) || !aligned(scales, 4) || !aligned(packed, 16)) return W4A16_EINVAL;
    const size_t sbytes = size_t(n) * size_t(k / kGroup) * 4;
    if (overlap(packed, pbytes, codes, cbytes) || overlap(packed, pbytes, scales, sbytes) ||
        (codes_out && overlap(codes, cbytes, scales, sbytes)))
        return W4A16_EINVAL;
    return W4A16_OK;
}

}  // namespace

extern "C" {

const char* w4a16_status_string(w4a16_status_t s) {
    switch (s) {
        case W4A16_OK: return "ok";
        case W4A16_EINVAL: return "invalid argument (shape, stride, pointer, alignment or overlap)";
        case W4A16_EUNSUPPORTED: return "unsupported request (dtype or path)";
        case W4A16_EWORKSPACE: return "workspace missing or too small";
        case W4A16_EHIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

size_t w4a16_packed_bytes(int64_t n, int64_t k) {
    if (!valid_nk(n, k)) return 0;
    return size_t(Layout(n, k).bytes());
}

size_t w8a16_packed_bytes(int64_t n, int64_t k) {
    if (!valid_nk(n, k)) return 0;
    return size_t(Layout(n, k, 8).bytes());
}

w4a16_status_t quantize_rtn_int4_g128(const void* w, w4a16_dtype_t w_dtype, int64_t n, int64_t k,
                                      int64_t ldw, uint8_t* codes, float* scales, void* stream) {
    const w4a16_status_t st =
        check_quantize(w, w_dtype, n, k, ldw, codes, size_t(n > 0 ? n : 0) * size_t(k > 0 ? k : 0) / 2, 4, scales);
    if (st != W4A16_OK || n == 0) return st;
    return from_hip(launch_quantize(w, int(w_dtype), n, k, ldw, codes, scales,
                                    static_cast<hipStream_t>(stream)));
}

w4a16_status_t quantize_rtn_int8_g128(const void* w, w4a16_dtype_t w_dtype, int64_t n, int64_t k,
                                      int64_t ldw, int8_t* codes, float* scales, void* stream) {
    const w4a16_status_t st =
        check_quantize(w, w_dtype, n, k, ldw, codes, size_t(n > 0 ? n : 0) * size_t(k > 0 ? k : 0), 8, scales);
    if (st != W4A16_OK || n == 0) return st;
    return from_hip(launch_quantize8(w, int(w_dtype), n, k, ldw, codes, scales,
                                     static_cast<hipStream_t>(stream)));
}

w4a16_status_t pack_weights(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                            void* packed, void* stream) {
    const w4a16_status_t st =
        check_pack(codes, size_t(n > 0 ? n : 0) * size_t(k > 0 ? k : 0) / 2, scales, n, k, packed,
                   w4a16_packed_bytes(n, k), false);
    if (st != W4A16_OK || n == 0) return st;
    return from_hip(launch_pack(codes, scales, n, k, packed, static_cast<hipStream_t>(stream)));
}

w4a16_status_t unpack_weights(const void* packed, int64_t n, int64_t k, uint8_t* codes, float* scales,
                              void* stream) {
    const w4a16_status_t st =
        check_pack(codes, size_t(n > 0 ? n : 0) * size_t(k > 0 ? k : 0) / 2, scales, n, k, packed,
                   w4a16_packed_bytes(n, k), true);
    if (st != W4A16_OK || n == 0) return st;
    return from_hip(launch_unpack(packed, n, k, codes, scales, static_cast<hipStream_t>(stream)));
}

w4a16_status_t pack_weights_int8(const int8_t* codes, const float* scales, int64_t n, int64_t k, void* packed,
                                 void* stream) {
    const w4a16_status_t st = check_pack(codes, size_t(n > 0 ? n : 0) * size_t(k > 0 ? k : 0), scales, n, k,
                                         packed, w8a16_packed_bytes(n, k), false);
    if (st != W4A16_OK || n == 0) return st;
    return from_hip(launch_pack8(codes, scales, n, k, packed, static_cast<hipStream_t>(stream)));
}

w4a16_status_t unpack_weights_int8(const void* packed, int64_t n, int64_t k, int8_t* codes, float* scales,
                                   void* stream) {
    const w4a16_status_t st = check_pack(codes, size_t(n > 0 ? n : 0) * size_t(k > 0 ? k : 0), scales, n, k,
                                         packed, w8a16_packed_bytes(n, k), true);
    if (st != W4A16_OK || n == 0) return st;
    return from_hip(launch_unpack8(packed, n, k, codes, scales, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

w4a16_status_t update_impl(int bits, void* packed, int64_t n, int64_t k, const void* update, int64_t ldu,
                           const void* mat1, const void* mat2, int64_t rank, w4a16_dtype_t update_dtype,
                           float alpha, float beta, const uint64_t* rounding_seed, void* stream) {
    if (update_dtype != W4A16_F32 && update_dtype != W4A16_BF16 && update_dtype != W4A16_F16)
        return W4A16_EUNSUPPORTED;
    if (!valid_nk(n, k) || rank < 0 || rank > kMaxRank) return W4A16_EINVAL;
    const bool dense = update != nullptr;
    if (dense == (rank > 0) || (dense && (mat1 || mat2)) || (!dense && (!mat1 || !mat2))) return W4A16_EINVAL;
    if (n == 0) return W4A16_OK;
    if (!packed || !aligned(packed, 16)) return W4A16_EINVAL;
    const size_t elem = update_dtype == W4A16_F32 ? 4 : 2;
    const size_t pbytes = bits == 8 ? w8a16_packed_bytes(n, k) : w4a16_packed_bytes(n, k);
    if (dense) {
        if (ldu < k || ldu > kMaxDim || !aligned(update, 16) || (size_t(ldu) * elem) % 16 != 0) return W4A16_EINVAL;
        if (overlap(packed, pbytes, update, span_bytes(n, k, ldu, elem))) return W4A16_EINVAL;
    } else {
        if (!aligned(mat2, 16) || !aligned(mat1, elem)) return W4A16_EINVAL;
        if (overlap(packed, pbytes, mat1, size_t(n) * size_t(rank) * elem) ||
            overlap(packed, pbytes, mat2, size_t(rank) * size_t(k) * elem))
            return W4A16_EINVAL;
    }
    const int dt = update_dtype == W4A16_F32 ? 0 : update_dtype == W4A16_BF16 ? kActBf16 : kActF16;
    return from_hip(launch_update(packed, n, k, update, ldu, mat1, mat2, rank, dt, alpha, beta,
                                  rounding_seed != nullptr, rounding_seed ? *rounding_seed : 0, bits,
                                  static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

w4a16_status_t w4a16_update_packed(void* packed, int64_t n, int64_t k, const void* update, int64_t ldu,
                                   const void* mat1, const void* mat2, int64_t rank, w4a16_dtype_t update_dtype,
                                   float alpha, float beta, const uint64_t* rounding_seed, void* stream) {
    return update_impl(4, packed, n, k, update, ldu, mat1, mat2, rank, update_dtype, alpha, beta, rounding_seed,
                       stream);
}

w4a16_status_t w8a16_update_packed(void* packed, int64_t n, int64_t k, const void* update, int64_t ldu,
                                   const void* mat1, const void* mat2, int64_t rank, w4a16_dtype_t update_dtype,
                                   float alpha, float beta, const uint64_t* rounding_seed, void* stream) {
    return update_impl(8, packed, n, k, update, ldu, mat1, mat2, rank, update_dtype, alpha, beta, rounding_seed,
                       stream);
}

}  // extern "C"

namespace {

w4a16_status_t shard_impl(int bits, const void* packed, int64_t n, int64_t k, int dim, int64_t start,
                          int64_t length, void* out, void* stream) {
    // a shard is a nonempty contiguous interval; input-feature shards hold
    // whole quantization groups
    if (!valid_nk(n, k) || n == 0 || (dim != 0 && dim != 1) || start < 0 || length <= 0) return W4A16_EINVAL;
    if (dim == 0 && start + length > n) return W4A16_EINVAL;
    if (dim == 1 && (start % kGroup != 0 || length % kGroup != 0 || start + length > k)) return W4A16_EINVAL;
    if (!packed || !out || !aligned(packed, 16) || !aligned(out, 16)) return W4A16_EINVAL;
    auto bytes = [bits](int64_t rows, int64_t cols) {
        return bits == 8 ? w8a16_packed_bytes(rows, cols) : w4a16_packed_bytes(rows, cols);
    };
    const size_t in_bytes = bytes(n, k);
    const size_t out_bytes = dim == 0 ? bytes(length, k) : bytes(n, length);
    if (overlap(packed, in_bytes, out, out_bytes)) return W4A16_EINVAL;
    return from_hip(launch_shard(packed, n, k, dim, start, length, out, bits, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

w4a16_status_t shard_packed_weights(const void* packed, int64_t n, int64_t k, int dim, int64_t start,
                                    int64_t length, void* out, void* stream) {
    return shard_impl(4, packed, n, k, dim, start, length, out, stream);
}

w4a16_status_t shard_packed_weights_int8(const void* packed, int64_t n, int64_t k, int dim, int64_t start,
                                         int64_t length, void* out, void* stream) {
    return shard_impl(8, packed, n, k, dim, start, length, out, stream);
}

w4a16_path_t w4a16_linear_choose_path(int64_t m, int64_t n, int64_t k) {
    // Measured (MI355X, graph replay, us): from M = 3 the MFMA contraction
    // beats v_dot2 (3 x 2048 x 16384: 8.2 vs 10.1); at M = 2 it does so on
    // layers above 8 M weights (2 x 32768 x 2048: 10.2 vs 10.5) and on narrow
    // ones, whose few tiles it splits over more workgroups (2 x 1024 x 4096:
    // 4.4 vs 5.1), while v_dot2 keeps the rest (2 x 2560 x 2048: 3.9 vs 4.3).
    // The small-M MFMA kernel finishes its K splits in-kernel and
    // wins over the mid-M kernel up to M = 16 on layers of <= 8 M weights
    // (16 x 2560 x 2048: 5.3 vs 8.1), up to M = 8 on layers of <= 16384
    // outputs (8 x 16384 x 2048: 7.8 vs 9.1) and up to M = 4 on wider ones
    // (8 x 32768 x 2048: 14.0 vs 12.9).  The mid-M kernel beats the GEMM
    // (whose few tiles need a K split and a reduce launch) on small layers up
    // to M = 512 (256 x 4096 x 1024: 9.3 vs 18.0); on layers of <= 32 M
    // weights up to M = 128 (128 x 16384 x 2048: 22.2 vs 22.8; 128 x 2048 x
    // 16384: 24.3 vs 27.0; at M = 160 the GEMM leads, 24.9 vs 29.0 and 30.7
    // vs 33.0); on larger ones up to M = 64 (64 x 32768 x 2048: 24.0 vs 25.3;
    // at M = 80 the GEMM leads, 25.6 vs 33.0; 96 x 4096 x 16384: 33.8 vs
    // 39.1).
    // With its x slice whole in LDS the mid-M kernel also takes M = 3-16 on
    // layers it covers without a K split (>= 16384 outputs, K <= 2048: 3 x
    // 32768 x 2048: 9.9 vs 10.7; 4 x 16384 x 2048: 6.6 vs 6.9; 8 x 16384 x
    // 2048: 6.7 vs 8.0), and wherever the small-M kernel's K split would
    // need the reduce launch (8 x 4096 x 16384: 12.7 vs 17.3); M = 2 is even
    // (2 x 32768 x 2048: 9.8 vs 9.7), and split layers stay with the small-M
    // kernel (4 x 2048 x 16384: 8.1 vs 9.1; 4 x 16384 x 4096: 11.2 vs 11.8).
    const bool small = n * k <= (int64_t(8) << 20);
    if (m <= 1 || (m == 2 && small && n >= 2048)) return W4A16_PATH_GEMV;
    if (m >= 3 && m <= 16 && k <= 2048 && n >= 16384) return W4A16_PATH_SKINNY;
    if (m <= 4 || (m <= 8 && n <= 16384) || (m <= 16 && small)) {
        // Direct plans (x operands loaded with the chunks, M > 4) split K
        // into at most a few exchange levels but put x through the vector
        // memory path four times per chunk: on layers of more than 32 M
        // weights the mid-M kernel, which shares x across its waves, leads
        // (M x N x K = 8 x 4096 x 16384: 13.3 vs 15.8 us; 8 x 16384 x 4096,
        // unsplit: 12.4 vs 13.6); on 8 x 2048 x 16384 the small-M kernel
        // leads, 8.8 vs 9.4.
        const MgemvPlan p = plan_mgemv(m < 16 ? m : 16, n, k, 4);
        const bool fits = p.direct ? n * k <= (int64_t(32) << 20) : p.splits == 1 || p.exchange;
        if (m <= 2 || small || fits) return W4A16_PATH_MGEMV;
    }
    const bool mid = n * k <= (int64_t(32) << 20);
    if (k > kGemmMaxLd || m <= 64 || (mid && m <= 128) || (small && m <= 512)) return W4A16_PATH_SKINNY;
    return W4A16_PATH_GEMM;
}

w4a16_path_t w8a16_linear_choose_path(int64_t m, int64_t n, int64_t k) {
    // Measured on INT8 weights (MI355X, us): the v_dot2 GEMV at M = 1 and at
    // M = 2 on layers of <= 8 M weights (2 x 2560 x 2048: 4.2 vs 4.6); the
    // small-M MFMA kernel at M = 2 on larger layers (2 x 32768 x 2048: 14.8
    // vs 15.1), at M = 3-8 (4 x 32768 x 2048: 15.1 vs 19.2; 8 x 2560 x 2048:
    // 5.1 vs 8.4 on the mid-M kernel) and at M = 9-16 on layers of <= 8 M
    // weights (16 x 4096 x 1024: 4.2 vs 6.8; on larger ones the mid-M kernel,
    // 16 x 16384 x 2048: 12.9 vs 14.2); the mid-M kernel above, the GEMM
    // from M = 65 on layers above 8 M weights (100 x 16384 x 2048: 31.7 vs
    // 43.9) and from M = 513 on smaller ones (256 x 4096 x 1024: 13.3 vs
    // 29.3; 1024 x 4096 x 1024: even).
    const bool small = n * k <= (int64_t(8) << 20);
    if (m <= 1 || (m == 2 && small)) return W4A16_PATH_GEMV;
    if (m <= 8 || (m <= 16 && small)) return W4A16_PATH_MGEMV;
    if (k > kGemmMaxLd || m <= 64 || (small && m <= 512)) return W4A16_PATH_SKINNY;
    return W4A16_PATH_GEMM;
}

}  // extern "C"

namespace {

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Byte offset of the materialised activated input in a GEMM + activation
// workspace: after the path's own workspace and never inside the zero
// header of exchange slots (an unsplit GEMM needs no workspace of its own).
size_t act_input_offset(w4a16_path_t path, int64_t m, int64_t n, int64_t k, int bits) {
    const size_t base = path_workspace(path, m, n, k, bits);
    return round_up(base > kSyncBytes ? base : kSyncBytes, 256);
}

// Workspace of one path with an activation: the large-M path materialises
// the activated input [m][k] after its own workspace.
size_t act_path_workspace(int act_fn, w4a16_path_t path, int64_t m, int64_t n, int64_t k, int bits) {
    const size_t base = path_workspace(path, m, n, k, bits);
    if (act_fn == kActFnNone || !is_gemm(path)) return base;
    return act_input_offset(path, m, n, k, bits) + size_t(m) * size_t(k) * 2;
}

size_t act_workspace_bytes(int act_fn, int64_t m, int64_t n, int64_t k, int bits) {
    if (m <= 0 || !valid_nk(n, k) || n == 0 || m > kMaxDim) return 0;
    size_t best = 0;
    const w4a16_path_t paths[4] = {W4A16_PATH_GEMV, W4A16_PATH_MGEMV, W4A16_PATH_SKINNY, W4A16_PATH_GEMM};
    for (w4a16_path_t p : paths) {
        const size_t b = act_path_workspace(act_fn, p, m, n, k, bits);
        best = b > best ? b : best;
    }
    return best;
}

// y = act(x) . dequant(packed)^T + bias on one kernel path (act_fn: ActFn;
// bits: 4 or 8, the packed weight's code width).
// launch == false: only the argument checks (the status a launching call
// would return before launching anything).
w4a16_status_t linear_impl(int bits, int act_fn, w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                           int64_t m, int64_t k, int64_t ldx, const void* packed, int64_t n, const void* bias,
                           void* y, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream,
                           bool launch = true) {
    if (act_dtype != W4A16_BF16 && act_dtype != W4A16_F16) return W4A16_EUNSUPPORTED;
    if (!valid_path(path)) return W4A16_EINVAL;
    if (!valid_nk(n, k) || m < 0 || m > kMaxDim) return W4A16_EINVAL;
    const int64_t xcols = act_fn == kActFnSwiglu ? 2 * k : k;  // SwiGLU rows hold [up | gate]
    if (ldx < xcols || ldx > kMaxDim || ldx % 8 != 0 || ldy < n || ldy > kMaxDim) return W4A16_EINVAL;
    if (m == 0 || n == 0) return W4A16_OK;
    if (!x || !packed || !y) return W4A16_EINVAL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 2) || (bias && !aligned(bias, 2)))
        return W4A16_EINVAL;
    // the GEMM reads its x tiles with 32-bit offsets: the row stride it sees
    // is ldx, or k for the materialised activation
    const int64_t gemm_ld = act_fn == kActFnNone ? ldx : k;
    if (path == W4A16_PATH_AUTO) {
        path = bits == 8 ? w8a16_linear_choose_path(m, n, k) : w4a16_linear_choose_path(m, n, k);
        if (path == W4A16_PATH_GEMM && gemm_ld > kGemmMaxLd) path = W4A16_PATH_SKINNY;
    }
    if (is_gemm(path) && gemm_ld > kGemmMaxLd) return W4A16_EUNSUPPORTED;

    const size_t xbytes = span_bytes(m, xcols, ldx, 2), ybytes = span_bytes(m, n, ldy, 2),
                 pbytes = bits == 8 ? w8a16_packed_bytes(n, k) : w4a16_packed_bytes(n, k),
                 bbytes = bias ? size_t(n) * 2 : 0;
    const size_t need = act_path_workspace(act_fn, path, m, n, k, bits);
    if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, packed, pbytes) ||
        overlap(y, ybytes, bias, bbytes) || overlap(y, ybytes, workspace, need))
        return W4A16_EINVAL;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return W4A16_EWORKSPACE;
        if (!aligned(workspace, 16)) return W4A16_EINVAL;
        if (overlap(workspace, need, x, xbytes) || overlap(workspace, need, packed, pbytes) ||
            overlap(workspace, need, bias, bbytes))
            return W4A16_EINVAL;
    }
    if (!launch) return W4A16_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int act = act_dtype == W4A16_BF16 ? kActBf16 : kActF16;
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    uint16_t* yp = static_cast<uint16_t*>(y);
    if (path == W4A16_PATH_GEMV) {
        // row blocks of at most 4; launches on one stream share the workspace
        for (int64_t r0 = 0; r0 < m; r0 += 4) {
            const int64_t mm = m - r0 < 4 ? m - r0 : 4;
            const hipError_t e = launch_gemv(xp + r0 * ldx, act, act_fn, bits, mm, k, ldx, packed, n, bias,
                                             yp + r0 * ldy, ldy, workspace, s);
            if (e != hipSuccess) return W4A16_EHIP;
        }
        return W4A16_OK;
    }
    if (path == W4A16_PATH_MGEMV) {
        for (int64_t r0 = 0; r0 < m; r0 += 16) {
            const int64_t mm = m - r0 < 16 ? m - r0 : 16;
            const hipError_t e = launch_mgemv(xp + r0 * ldx, act, act_fn, bits, mm, k, ldx, packed, n, bias,
                                              yp + r0 * ldy, ldy, workspace, s);
            if (e != hipSuccess) return W4A16_EHIP;
        }
        return W4A16_OK;
    }
    if (is_gemm(path)) {
        const bool sk = path == W4A16_PATH_GEMM_STREAMK;
        if (act_fn == kActFnNone)
            return from_hip(launch_gemm(x, act, bits, m, k, ldx, packed, n, bias, y, ldy, workspace, sk, s));
        void* xa = static_cast<uint8_t*>(workspace) + act_input_offset(path, m, n, k, bits);
        const hipError_t e = launch_activate(x, act, act_fn, m, k, ldx, xa, s);
        if (e != hipSuccess) return W4A16_EHIP;
        return from_hip(launch_gemm(xa, act, bits, m, k, k, packed, n, bias, y, ldy, workspace, sk, s));
    }
    return from_hip(launch_skinny(x, act, act_fn, bits, m, k, ldx, packed, n, bias, y, ldy, workspace, s));
}

}  // namespace

namespace w4a16 {

w4a16_status_t check_linear(const void* x, w4a16_dtype_t act_dtype, int64_t m, int64_t k, int64_t ldx,
                            const void* packed, int64_t n, const void* bias, void* y, int64_t ldy,
                            void* workspace, size_t workspace_bytes) {
    return linear_impl(4, kActFnNone, W4A16_PATH_AUTO, x, act_dtype, m, k, ldx, packed, n, bias, y, ldy, workspace,
                       workspace_bytes, nullptr, false);
}

}  // namespace w4a16

extern "C" {

size_t w4a16_linear_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    return act_workspace_bytes(kActFnNone, m, n, k, 4);
}

w4a16_status_t w4a16_linear_explain(int bits, w4a16_act_t act, w4a16_path_t path, int64_t m, int64_t n, int64_t k,
                                    w4a16_plan_t* plan) {
    if (!plan || (bits != 4 && bits != 8)) return W4A16_EINVAL;
    if (act != W4A16_ACT_NONE && act != W4A16_ACT_SWIGLU && act != W4A16_ACT_GELU_TANH) return W4A16_EINVAL;
    if (!valid_path(path)) return W4A16_EINVAL;
    if (!valid_nk(n, k) || m < 0 || m > kMaxDim) return W4A16_EINVAL;
    *plan = w4a16_plan_t{};
    // rows contiguous: the GEMM sees a row stride of k (also for an activation,
    // which it materialises with stride k)
    if (path == W4A16_PATH_AUTO) {
        path = bits == 8 ? w8a16_linear_choose_path(m, n, k) : w4a16_linear_choose_path(m, n, k);
        if (path == W4A16_PATH_GEMM && k > kGemmMaxLd) path = W4A16_PATH_SKINNY;
    }
    plan->path = path;
    if (m == 0 || n == 0) return W4A16_OK;
    const int fn = int(act);
    PlanInfo info{};
    int64_t launches = 1;
    switch (path) {
        case W4A16_PATH_GEMV: info = describe_gemv(m < 4 ? m : 4, n, k, bits); launches = ceil_div(m, 4); break;
        case W4A16_PATH_MGEMV: info = describe_mgemv(m < 16 ? m : 16, n, k, bits, fn); launches = ceil_div(m, 16); break;
        case W4A16_PATH_SKINNY: info = describe_skinny(m, n, k, bits, fn); break;
        default: info = describe_gemm(m, n, k, bits, path == W4A16_PATH_GEMM_STREAMK); break;
    }
    plan->waves = info.waves;
    plan->tile_m = info.tile_m;
    plan->tile_n = info.tile_n;
    plan->splits = info.splits;
    plan->groups_per_split = info.gps;
    plan->workgroups = info.workgroups;
    plan->launches = launches * (info.reduce ? 2 : 1) + (is_gemm(path) && fn != kActFnNone ? 1 : 0);
    plan->stream_k = info.stream_k ? 1 : 0;
    plan->workspace_bytes = uint64_t(act_path_workspace(fn, path, m, n, k, bits));
    return W4A16_OK;
}

size_t w4a16_linear_act_workspace_bytes(w4a16_act_t act, int64_t m, int64_t n, int64_t k) {
    if (act != W4A16_ACT_NONE && act != W4A16_ACT_SWIGLU && act != W4A16_ACT_GELU_TANH) return 0;
    return act_workspace_bytes(int(act), m, n, k, 4);
}

size_t w8a16_linear_workspace_bytes(w4a16_act_t act, int64_t m, int64_t n, int64_t k) {
    if (act != W4A16_ACT_NONE && act != W4A16_ACT_SWIGLU && act != W4A16_ACT_GELU_TANH) return 0;
    return act_workspace_bytes(int(act), m, n, k, 8);
}

w4a16_status_t w8a16_linear(w4a16_act_t act, w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                            int64_t m, int64_t k, int64_t ldx, const void* packed, int64_t n, const void* bias,
                            void* y, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
    if (act != W4A16_ACT_NONE && act != W4A16_ACT_SWIGLU && act != W4A16_ACT_GELU_TANH) return W4A16_EINVAL;
    return linear_impl(8, int(act), path, x, act_dtype, m, k, ldx, packed, n, bias, y, ldy, workspace,
                       workspace_bytes, stream);
}

w4a16_status_t w4a16_linear_with_path(w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                                      int64_t m, int64_t k, int64_t ldx, const void* packed,
                                      int64_t n, const void* bias, void* y, int64_t ldy,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    return linear_impl(4, kActFnNone, path, x, act_dtype, m, k, ldx, packed, n, bias, y, ldy, workspace,
                       workspace_bytes, stream);
}

w4a16_status_t w4a16_linear(const void* x, w4a16_dtype_t act_dtype, int64_t m, int64_t k, int64_t ldx,
                            const void* packed, int64_t n, const void* bias, void* y, int64_t ldy,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return linear_impl(4, kActFnNone, W4A16_PATH_AUTO, x, act_dtype, m, k, ldx, packed, n, bias, y, ldy,
                       workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_linear_act(w4a16_act_t act, w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                                int64_t m, int64_t k, int64_t ldx, const void* packed, int64_t n,
                                const void* bias, void* y, int64_t ldy, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (act != W4A16_ACT_NONE && act != W4A16_ACT_SWIGLU && act != W4A16_ACT_GELU_TANH) return W4A16_EINVAL;
    return linear_impl(4, int(act), path, x, act_dtype, m, k, ldx, packed, n, bias, y, ldy, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
