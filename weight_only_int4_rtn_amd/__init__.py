"""W4A16 quantized linear layer for AMD MI355X (gfx950).

Weights are round-to-nearest quantized to INT4 with one FP32 scale per group
of 128 along K when they are loaded; activations stay BF16/FP16; the layer
computes y = x . dequant(Wq, s)^T (+ bias) in hand-written HIP kernels
behind the C ABI of ``include/w4a16.h``.

    codes, scales = quantize(w)          # load time, w [n, k] on the GPU
    packed = pack(codes, scales)         # load time
    y = linear(x, packed, n, bias)       # every forward step
    y = linear(up_gate, packed_down, n, act=Act.SWIGLU)   # activation fused into the input

INT8 weights (W8A16) take the same calls with the 8-bit quantizer:

    codes8, scales8 = quantize_int8(w)
    packed8 = pack_int8(codes8, scales8)
    y = linear(x, packed8, n, bias, bits=8)
"""
import torch  # noqa: F401  (load torch's HIP runtime before the library)

from ._binding import (  # noqa: F401
    GROUP,
    Act,
    Path,
    W4A16ArgumentError,
    W4A16Error,
    W4A16LaunchError,
    choose_path,
    explain,
    lib,
    linear,
    linear_noalloc,
    pack,
    pack_int8,
    packed_bytes,
    quantize,
    quantize_int8,
    shard,
    status_string,
    unpack,
    unpack_int8,
    update_,
    workspace_bytes,
)
