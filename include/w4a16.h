/*
 * w4a16.h -- C ABI of the W4A16 quantized linear layer for AMD MI355X (gfx950).
 *
 * The layer, as the pages define it:
 *   - weights are quantized once, when a FP16/BF16/FP32 checkpoint is loaded,
 *     by round-to-nearest to INT4 with one scale per group of 128 weights;
 *     activations stay BF16 or FP16 ("Kernel dispatch and Humming
 *     quantization in PhyAI", section "Humming makes the separation useful");
 *   - a quantized weight carries its own packed layout, which a plain 16-bit
 *     GEMM cannot execute (same page and section);
 *   - y = x . dequant(Wq, s)^T + bias, weight [out_features, in_features],
 *     input [..., in_features], output [..., out_features] ("Piper Kernels",
 *     section "ConvRot INT8"); scales and bias are applied in FP32 before the
 *     one final conversion to the output dtype ("Piper Kernels", section
 *     "NVFP4 construction").
 *
 * Readings fixed by this library where the pages are silent: symmetric codes
 * without a zero point; scale s = max|w| / 7 over 128 consecutive weights of
 * one output row (one correctly rounded FP32 division); code
 * q = clamp(round_half_even(fl32(w / s)), -8, 7), and q = 0 where s == 0.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; every call is asynchronous on `stream` (a
 *     hipStream_t; NULL is the null stream).
 *   - The caller allocates and owns every buffer.  The library never
 *     allocates, frees or synchronizes, and never reads device contents on
 *     the host ("Piper Kernels", section "Validation contract"): arguments
 *     are checked from their values (shapes, dtypes, alignment, sizes) only,
 *     and a failed check returns an error before anything is launched.
 *   - Tensor contents are caller preconditions: NaN or Inf in weights,
 *     activations or bias give unspecified results and no error.
 *   - All calls can be captured into a HIP graph.
 *   - Calls on different streams may run concurrently as long as they do not
 *     share output buffers or a workspace.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_EINVAL = 1,        /* bad shape, stride, pointer, alignment or overlap */
    W4A16_EUNSUPPORTED = 2,  /* valid request the library does not implement (e.g. dtype) */
    W4A16_EWORKSPACE = 3,    /* workspace missing or smaller than required */
    W4A16_EHIP = 4           /* the HIP runtime reported an error at launch */
} w4a16_status_t;

typedef enum {
    W4A16_F32 = 0,
    W4A16_BF16 = 1,
    W4A16_F16 = 2
} w4a16_dtype_t;

/* Kernel families w4a16_linear chooses between (by M, N, K). */
typedef enum {
    W4A16_PATH_AUTO = 0,    /* let the library choose */
    W4A16_PATH_GEMV = 1,    /* small M: VALU v_dot2 products, split-K, cross-lane reductions */
    W4A16_PATH_MGEMV = 2,   /* small M: the same weight stream contracted on MFMA */
    W4A16_PATH_SKINNY = 3,  /* mid M: register-dequantized MFMA, x tiles through LDS */
    W4A16_PATH_GEMM = 4,    /* large M: LDS-staged dequantized tiles into MFMA */
    W4A16_PATH_GEMM_STREAMK = 5 /* the large-M kernel with a stream-K decomposition (explicit only:
                                   slower than the planner's cut on the shapes measured) */
} w4a16_path_t;

/*
 * Activation applied to a linear layer's input before the product
 * ("Piper Kernels", section "ConvRot INT8": an activated linear takes
 * activation_fn "swiglu", whose input rows are [up | gate] of twice the
 * layer's in_features and give up * silu(gate), or "gelu_tanh", the
 * tanh-approximate GELU of the input).  Evaluated in FP32 and rounded once to
 * the activation dtype (nearest even) before it enters the product.
 */
typedef enum {
    W4A16_ACT_NONE = 0,      /* y = x . W^T + b */
    W4A16_ACT_SWIGLU = 1,    /* y = (up * silu(gate)) . W^T + b, x rows = [up | gate], silu(g) = g / (1 + e^-g) */
    W4A16_ACT_GELU_TANH = 2  /* y = gelu(x) . W^T + b, gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))) */
} w4a16_act_t;

/* Group size along K: one FP32 scale per 128 consecutive weights of a row. */
#define W4A16_GROUP 128

/*
 * Round-to-nearest INT4 quantization with one FP32 scale per group of 128
 * ("Kernel dispatch and Humming quantization in PhyAI", section "Humming
 * makes the separation useful"; the readings listed at the top of this file).
 *
 *   w       device, [n][ldw] elements of w_dtype (F32, BF16 or F16), row-major
 *           [out_features, in_features]; 16-byte aligned; ldw * element size
 *           a multiple of 16 bytes.  16-bit weights are widened to FP32
 *           exactly before quantization.
 *   n, k    rows and columns; n >= 0, k > 0, k % 128 == 0, ldw >= k.
 *   codes   device, [n][k/2] bytes, the canonical layout: byte j of a row
 *           holds the code of column 2j in its low nibble and of column 2j+1
 *           in its high nibble, 4-bit two's complement; 4-byte aligned.
 *   scales  device, [n][k/128] FP32, row-major; 4-byte aligned.
 * Returns W4A16_OK (also for n == 0, which launches nothing), W4A16_EINVAL,
 * W4A16_EUNSUPPORTED (unknown dtype) or W4A16_EHIP.
 */
w4a16_status_t quantize_rtn_int4_g128(const void* w, w4a16_dtype_t w_dtype, int64_t n, int64_t k,
                                      int64_t ldw, uint8_t* codes, float* scales, void* stream);

/*
 * Size in bytes of the packed weight for an [n][k] layer (k % 128 == 0),
 * or 0 for invalid sizes.  The packed layout is the library's own execution
 * format: a quantized weight carries a layout of its own that a plain 16-bit
 * GEMM cannot execute ("Kernel dispatch and Humming quantization in PhyAI",
 * section "Humming makes the separation useful"), the physical form of a
 * weight whose semantic form is its codes and scales ("量化概述", section
 * "量化").  It is not a storage format: store codes and scales, and pack
 * after loading.  Pure host arithmetic; no error status (0 marks bad sizes).
 */
size_t w4a16_packed_bytes(int64_t n, int64_t k);

/*
 * Canonical codes and scales -> the packed execution layout.
 *   codes   device, [n][k/2] canonical bytes (see quantize_rtn_int4_g128); 4-byte aligned.
 *   scales  device, [n][k/128] FP32; 4-byte aligned.
 *   packed  device, w4a16_packed_bytes(n, k) bytes; 16-byte aligned; must not
 *           overlap codes or scales.
 * Codes are taken as given (any 4-bit value, including -8).  Returns
 * W4A16_OK, W4A16_EINVAL or W4A16_EHIP.
 */
w4a16_status_t pack_weights(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                            void* packed, void* stream);

/*
 * Inverse of pack_weights: packed layout -> canonical codes and scales,
 * bit-exact (the lowering from the semantic to the physical form loses
 * nothing, "量化概述", section "量化"; nibble and packed-pair order are
 * preserved, "Piper Kernels", section "NVFP4 construction").
 *   packed  device, w4a16_packed_bytes(n, k) bytes from pack_weights; 16-byte aligned.
 *   codes   device output, [n][k/2] canonical bytes; 4-byte aligned.
 *   scales  device output, [n][k/128] FP32; 4-byte aligned; codes and scales
 *           must not overlap each other or packed.
 * n == 0 is a no-op.  Returns W4A16_OK, W4A16_EINVAL or W4A16_EHIP.
 */
w4a16_status_t unpack_weights(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                              float* scales, void* stream);

/*
 * In-place update of a packed [n][k] weight ("Piper Kernels", sections
 * "ConvRot INT8" -- add_ / addmm_ requantize the updated weight; an unsigned
 * 64-bit rounding_seed selects stochastic rounding without changing the
 * scales, none selects nearest rounding -- and "Stochastic quantization" --
 * one of the two adjacent codes with probability proportional to distance,
 * values outside the code range and exact hits never perturbed, draws by
 * logical element offset):
 *   W' = beta * dequant(W) + alpha * U
 * with U the dense update [n][ldu] (update != NULL, rank == 0) or the
 * low-rank product mat1 [n][rank] @ mat2 [rank][k] (update == NULL,
 * 1 <= rank <= 65536), all of update_dtype (F32, BF16 or F16), row-major.
 * Every step is one FP32 operation: d = fl32(q * s); U widened to FP32, or
 * p = fma(mat1[n][r], mat2[r][k], p) over r ascending from 0; w' =
 * fma(alpha, p, fl32(beta * d)).  W' is then quantized with the rules of
 * quantize_rtn_int4_g128 (scale amax / 7 per group); with a seed, an
 * interior quotient v (-8 <= floor(v) <= 6) becomes floor(v) + 1 exactly when
 * u < v - floor(v), u = (SplitMix64 output e+1 of the seed) >> 40, times
 * 2^-24, e = n * k_total + k the element's row-major offset (SplitMix64:
 * Steele, Lea and Flood, OOPSLA 2014).  Results are identical from run to
 * run and independent of the launch.
 *   packed   device, from pack_weights, 16-byte aligned; updated in place.
 *   update   device, 16-byte aligned, ldu >= k, ldu * element size a
 *            multiple of 16 bytes.
 *   mat1     device, element-aligned; mat2 device, 16-byte aligned.
 *   rounding_seed  host pointer to the seed, or NULL for nearest rounding.
 * The update operands must not overlap packed.  n == 0 is a no-op.  Returns
 * W4A16_OK, W4A16_EINVAL, W4A16_EUNSUPPORTED (update_dtype) or W4A16_EHIP.
 * Repeated requantization is lossy.
 */
w4a16_status_t w4a16_update_packed(void* packed, int64_t n, int64_t k, const void* update, int64_t ldu,
                                   const void* mat1, const void* mat2, int64_t rank,
                                   w4a16_dtype_t update_dtype, float alpha, float beta,
                                   const uint64_t* rounding_seed, void* stream);

/*
 * A shard of an already packed [n][k] weight, without requantizing ("Piper
 * Kernels", section "NVFP4 construction", partitioning an already quantized
 * weight: packed data is copied, nibble order and scales are preserved, each
 * shard owns its storage, a shard is a nonempty contiguous interval, and
 * input-channel shards align to the format's blocks).
 *   dim 0 (output features): rows [start, start + length), any start;
 *          out = packed [length][k], w4a16_packed_bytes(length, k) bytes.
 *   dim 1 (input features): columns [start, start + length), both multiples
 *          of 128 (whole quantization groups), length > 0;
 *          out = packed [n][length], w4a16_packed_bytes(n, length) bytes.
 * unpack_weights(out) equals the same rows / columns of unpack_weights(packed),
 * and out is byte-identical to pack_weights of those canonical rows / columns.
 * packed and out are device pointers, 16-byte aligned, and must not overlap.
 * n == 0, length <= 0 or an interval outside the weight give W4A16_EINVAL.
 * Returns W4A16_OK, W4A16_EINVAL or W4A16_EHIP.
 */
w4a16_status_t shard_packed_weights(const void* packed, int64_t n, int64_t k, int dim, int64_t start,
                                    int64_t length, void* out, void* stream);

/*
 * Workspace bytes w4a16_linear needs for an [m][k] x [n][k] product, for every
 * kernel path but W4A16_PATH_GEMM_STREAMK, whose need w4a16_linear_explain
 * reports (0 if none, also for invalid sizes).  The caller owns it: the
 * library allocates nothing and reads nothing back ("Piper Kernels", section
 * "Validation contract": no temporary device allocations, no
 * synchronization, nothing that would stop graph capture; "Kernel dispatch
 * and Humming quantization in PhyAI", section "A kernel choice belongs to a
 * workload": a kernel used inside a graph must support capture).  A K split needs it: a 1 MiB header of exchange
 * slots through which the small-M kernels add the parts' sums inside one
 * launch, then FP32 partial sums that a second small kernel adds in split
 * order (no floating-point atomics either way); a stream-K launch keeps one
 * counter per output tile in the header and its FP32 tile sums after it.  The caller zero-fills a
 * workspace once, before its first use; every call leaves the header zero
 * again, so a workspace is reused without clearing (also by calls of other
 * shapes and paths).  Two calls that may run at the same time must not share
 * a workspace.
 */
size_t w4a16_linear_workspace_bytes(int64_t m, int64_t n, int64_t k);

/*
 * y[m][n] = x[m][k] . dequant(packed)^T + bias[n], with
 * dequant(q, s)[n][k] = q[n][k] * s[n][k / 128]; FP32 accumulation; the bias
 * is added in FP32 once; the result is rounded to act_dtype (nearest even).
 * The W4A16 layer: INT4 weights with one scale per group of 128, BF16 or
 * FP16 activations ("Kernel dispatch and Humming quantization in PhyAI",
 * section "Humming makes the separation useful"); weight [out_features,
 * in_features], input [..., in_features], output [..., out_features] in the
 * input's dtype ("Piper Kernels", section "ConvRot INT8"); scales and bias
 * in FP32 before the one final 16-bit conversion ("Piper Kernels", section
 * "NVFP4 construction").
 *
 *   x         device, [m][ldx] of act_dtype (BF16 or F16), 16-byte aligned, ldx >= k,
 *             ldx % 8 == 0.
 *   m, k      m >= 0; k > 0, k % 128 == 0 (the layer's in_features).
 *   packed    device, from pack_weights for (n, k); 16-byte aligned.
 *   n         out_features, n >= 0.
 *   bias      device [n] of act_dtype, or NULL; 2-byte aligned.
 *   y         device, [m][ldy] of act_dtype, ldy >= n, 2-byte aligned; must not
 *             overlap x, packed, bias or workspace.
 *   workspace device, >= w4a16_linear_workspace_bytes(m, n, k) bytes, 16-byte
 *             aligned, zero-filled before its first use and then only
 *             passed to these calls (may be NULL when that size is 0).
 * m == 0 or n == 0 returns W4A16_OK and launches nothing.  Returns W4A16_OK,
 * W4A16_EINVAL, W4A16_EUNSUPPORTED (act_dtype), W4A16_EWORKSPACE or W4A16_EHIP.
 * The result is bit-identical from run to run (no floating-point atomics).
 */
w4a16_status_t w4a16_linear(const void* x, w4a16_dtype_t act_dtype, int64_t m, int64_t k,
                            int64_t ldx, const void* packed, int64_t n, const void* bias,
                            void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * w4a16_linear with an explicit kernel path (W4A16_PATH_AUTO behaves exactly
 * like w4a16_linear).  Every path accepts every valid m; the automatic choice
 * is the fast one.  For tests and measurements of each kernel.  The GEMM path
 * addresses its x tiles with 32-bit offsets and returns W4A16_EUNSUPPORTED for
 * ldx > 4194304 (2^22); the automatic choice then takes the SKINNY path.
 * W4A16_PATH_GEMM_STREAMK runs the GEMM kernel with a stream-K decomposition
 * whatever the planner would choose ("Kernel dispatch and Humming
 * quantization in PhyAI", introduction: a kernel cut that suits one workload
 * can be a poor one for another): the tiles x 128-column groups of work are
 * cut into runs of equal length, one workgroup each, and the runs that share
 * a tile add their FP32 sums in K order through the workspace, the last one
 * to finish a tile storing it (reproducible, no waiting between
 * workgroups).  Same limits as the GEMM path; its workspace is the one
 * w4a16_linear_explain reports for it.  The automatic choice never takes
 * it: on MI355X it measured slower than the planner's equal K split on every
 * shape tried (the fix-up's slot round trips fall on the launch's tail).
 */
w4a16_status_t w4a16_linear_with_path(w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                                      int64_t m, int64_t k, int64_t ldx, const void* packed,
                                      int64_t n, const void* bias, void* y, int64_t ldy,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes w4a16_linear_act needs (0 if none; 0 for an unknown act).
 * Same header rules as w4a16_linear_workspace_bytes; with an activation the
 * large-M path also keeps the activated input, m * k 16-bit values, there
 * (after the header and the GEMM's own partial sums).
 */
size_t w4a16_linear_act_workspace_bytes(w4a16_act_t act, int64_t m, int64_t n, int64_t k);

/*
 * y[m][n] = act(x)[m][k] . dequant(packed)^T + bias[n]: a linear layer with
 * its input activation fused ("Piper Kernels", section "ConvRot INT8"; the
 * down projection of an FFN).  The small- and mid-M paths apply the
 * activation while they stage x (one launch); the large-M path materialises
 * the activated input in the workspace first, with the same arithmetic.
 *
 *   act       W4A16_ACT_NONE (exactly w4a16_linear_with_path), SWIGLU or
 *             GELU_TANH; anything else gives W4A16_EINVAL.
 *   path      as for w4a16_linear_with_path (W4A16_PATH_AUTO: the library
 *             chooses; the GEMM path then requires k <= 2^22 instead of ldx).
 *   x         device, [m][ldx] of act_dtype, 16-byte aligned, ldx % 8 == 0;
 *             SWIGLU: each row holds up in columns [0, k) and gate in
 *             [k, 2k), ldx >= 2k; GELU_TANH / NONE: ldx >= k.
 *   workspace >= w4a16_linear_act_workspace_bytes(act, m, n, k) bytes.
 * Every other argument, the no-op cases, the overlap rules (y against all of
 * x's rows) and the status codes are those of w4a16_linear.
 */
w4a16_status_t w4a16_linear_act(w4a16_act_t act, w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                                int64_t m, int64_t k, int64_t ldx, const void* packed, int64_t n,
                                const void* bias, void* y, int64_t ldy, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * w4a16_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (minus the workspace), checks, kernels and bit-identical
 * results as w4a16_linear; the workspace is instead a fixed array of
 * W4A16_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends.  The call allocates nothing.  Its first call on a
 * device looks the array's address up (hipGetSymbolAddress) and launches one
 * small kernel on `stream` that zeroes the array's header.
 *   - A call whose plan needs more workspace than the array holds returns
 *     W4A16_EWORKSPACE before launching anything (the limit is a property
 *     of the shape: w4a16_linear with a caller workspace takes any size).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that may overlap on one GPU (several streams,
 *     several host threads) race and must be serialised by the caller.
 * Returns the statuses of w4a16_linear (W4A16_EUNSUPPORTED also for a device
 * index of 64 or more).
 */
#define W4A16_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
w4a16_status_t w4a16_linear_noalloc(const void* x, w4a16_dtype_t act_dtype, int64_t m, int64_t k, int64_t ldx,
                                    const void* packed, int64_t n, const void* bias, void* y, int64_t ldy,
                                    void* stream);

/*
 * The plan of one linear call: which kernel family runs and how its work is
 * cut.  The library plans from (bits, act, m, n, k) alone, with no tuning
 * and no state, so the same sizes always take the same plan and results are
 * reproducible.
 */
typedef struct {
    int32_t path;              /* the w4a16_path_t the call takes (never W4A16_PATH_AUTO) */
    int32_t waves;             /* waves of 64 lanes per workgroup of the main kernel */
    int32_t tile_m, tile_n;    /* x rows and output columns one workgroup computes */
    int32_t splits;            /* parts K is split into (1: none) */
    int32_t groups_per_split;  /* 128-column groups per part */
    int64_t workgroups;        /* workgroups of one launch of the main kernel */
    int64_t launches;          /* kernel launches of the whole call */
    uint64_t workspace_bytes;  /* workspace this plan needs (<= w4a16_linear_act_workspace_bytes) */
    int32_t stream_k;          /* 1: stream-K (workgroups = runs of equal length over tiles x groups;
                                  splits = the most runs sharing a tile, groups_per_split = the
                                  longest run) */
    int32_t reserved;
} w4a16_plan_t;

/*
 * Explains the plan w4a16_linear_act / w8a16_linear (bits 4 / 8) would run
 * for an [m][k] input with contiguous rows and an [n][k] weight on `path`
 * (W4A16_PATH_AUTO: the library's choice).  Pure host computation, no
 * launch; the dispatcher can explain its decision ("Kernel dispatch and
 * Humming quantization in PhyAI", section "Put deployment choices in a
 * policy").  m == 0 or n == 0 report the path with zero launches.
 *   plan  host pointer, filled on W4A16_OK.
 * Returns W4A16_OK or W4A16_EINVAL (bits, act, path, sizes, NULL plan).
 */
w4a16_status_t w4a16_linear_explain(int bits, w4a16_act_t act, w4a16_path_t path, int64_t m, int64_t n, int64_t k,
                                    w4a16_plan_t* plan);

/* The path w4a16_linear would take for these sizes (never W4A16_PATH_AUTO). */
w4a16_path_t w4a16_linear_choose_path(int64_t m, int64_t n, int64_t k);

/* ------------------------------------------------------------------------
 * W8A16: INT8 weights.  The same integration lists INT8 beside INT4 among
 * its weight schemes ("Kernel dispatch and Humming quantization in PhyAI",
 * section "Choose precision by layer and hardware"); the method is the same
 * round-to-nearest quantizer with one FP32 scale per group of 128 along K,
 * with the 8-bit code range.
 * ------------------------------------------------------------------------ */

/*
 * Round-to-nearest INT8 quantization, group 128:
 *   s[n][g] = fl32(max_{k in group g} |w[n][k]| / 127)      (FP32 division)
 *   q[n][k] = clamp(round_half_even(fl32(w[n][k] / s)), -128, 127), 0 if s == 0
 * (-128 is never produced).  Arguments as for quantize_rtn_int4_g128, except
 *   codes   device, [n][k] int8, one two's-complement code per byte; 8-byte
 *           aligned.
 * Returns W4A16_OK (also for n == 0), W4A16_EINVAL, W4A16_EUNSUPPORTED or
 * W4A16_EHIP.
 */
w4a16_status_t quantize_rtn_int8_g128(const void* w, w4a16_dtype_t w_dtype, int64_t n, int64_t k,
                                      int64_t ldw, int8_t* codes, float* scales, void* stream);

/* Size in bytes of the packed INT8 weight for an [n][k] layer (0 for invalid sizes). */
size_t w8a16_packed_bytes(int64_t n, int64_t k);

/*
 * INT8 canonical codes [n][k] and scales [n][k/128] -> the packed INT8
 * execution layout (w8a16_packed_bytes(n, k) bytes), and its exact inverse.
 * codes and scales 4-byte aligned, packed 16-byte aligned, no overlaps.
 * Returns W4A16_OK, W4A16_EINVAL or W4A16_EHIP.
 */
w4a16_status_t pack_weights_int8(const int8_t* codes, const float* scales, int64_t n, int64_t k, void* packed,
                                 void* stream);
w4a16_status_t unpack_weights_int8(const void* packed, int64_t n, int64_t k, int8_t* codes, float* scales,
                                   void* stream);

/*
 * A shard of an already packed INT8 [n][k] weight: the rules, arguments and
 * status codes of shard_packed_weights, with w8a16_packed_bytes sizes; the
 * shard equals pack_weights_int8 of the same canonical rows / columns.
 */
w4a16_status_t shard_packed_weights_int8(const void* packed, int64_t n, int64_t k, int dim, int64_t start,
                                         int64_t length, void* out, void* stream);

/*
 * In-place update of a packed INT8 [n][k] weight (from pack_weights_int8):
 * the arithmetic, arguments and status codes of w4a16_update_packed, with
 * the INT8 quantizer (scale amax / 127, codes [-128, 127]) and, with a seed,
 * stochastic rounding where -128 <= floor(v) <= 126 ("Piper Kernels",
 * section "ConvRot INT8": one of the two adjacent INT8 codes).
 */
w4a16_status_t w8a16_update_packed(void* packed, int64_t n, int64_t k, const void* update, int64_t ldu,
                                   const void* mat1, const void* mat2, int64_t rank,
                                   w4a16_dtype_t update_dtype, float alpha, float beta,
                                   const uint64_t* rounding_seed, void* stream);

/* Workspace bytes w8a16_linear needs (0 if none; 0 for an unknown act); header rules as above. */
size_t w8a16_linear_workspace_bytes(w4a16_act_t act, int64_t m, int64_t n, int64_t k);

/*
 * y[m][n] = act(x)[m][k] . dequant(packed)^T + bias[n] for a packed INT8
 * weight (from pack_weights_int8): the arithmetic, arguments, activations,
 * no-op cases, overlap rules and status codes of w4a16_linear_act.  Paths:
 * W4A16_PATH_AUTO, W4A16_PATH_GEMV (row blocks of 4), W4A16_PATH_MGEMV (row
 * blocks of 16), W4A16_PATH_SKINNY, W4A16_PATH_GEMM and W4A16_PATH_GEMM_STREAMK
 * (any m; the GEMM with the row-stride limit of w4a16_linear_with_path).
 * workspace >= w8a16_linear_workspace_bytes(act, m, n, k) bytes.
 */
w4a16_status_t w8a16_linear(w4a16_act_t act, w4a16_path_t path, const void* x, w4a16_dtype_t act_dtype,
                            int64_t m, int64_t k, int64_t ldx, const void* packed, int64_t n, const void* bias,
                            void* y, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* The path w8a16_linear takes for these sizes with W4A16_PATH_AUTO. */
w4a16_path_t w8a16_linear_choose_path(int64_t m, int64_t n, int64_t k);

/*
 * Static, human-readable text for a status code ("unknown status" for values
 * outside w4a16_status_t).  Errors cross the ABI as status codes only, and
 * each names a concrete reason ("Kernel dispatch and Humming quantization in
 * PhyAI", section "Put deployment choices in a policy": an unsupported
 * layout or a capture restriction becomes a concrete diagnosis).  The
 * returned string is owned by the library; never NULL.
 */
const char* w4a16_status_string(w4a16_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
