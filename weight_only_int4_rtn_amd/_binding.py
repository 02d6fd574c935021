"""ctypes binding over the C ABI (include/w4a16.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory and the current stream.  The library must be
loaded after torch so both share torch's HIP runtime.
"""
from __future__ import annotations

import ctypes
import enum
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")
GROUP = 128
NOALLOC_SCRATCH_BYTES = 32 << 20  # W4A16_NOALLOC_SCRATCH_BYTES of include/w4a16.h

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
F32, BF16, F16 = 0, 1, 2


class Path(enum.IntEnum):
    AUTO = 0
    GEMV = 1
    MGEMV = 2
    SKINNY = 3
    GEMM = 4
    GEMM_STREAMK = 5


class Act(enum.IntEnum):
    """Activation fused into a linear's input (w4a16_act_t)."""
    NONE = 0
    SWIGLU = 1      # input rows [up | gate] (2k values) -> up * silu(gate)
    GELU_TANH = 2   # tanh-approximate GELU of the input


class W4A16Error(Exception):
    """A status other than W4A16_OK from the C ABI; ``status`` holds it."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class W4A16ArgumentError(W4A16Error, ValueError):
    """W4A16_EINVAL, W4A16_EUNSUPPORTED or W4A16_EWORKSPACE: the request was
    rejected from its arguments before anything was launched."""


class W4A16LaunchError(W4A16Error, RuntimeError):
    """W4A16_EHIP: the HIP runtime reported an error at launch."""


class PlanT(ctypes.Structure):
    """w4a16_plan_t"""
    _fields_ = [("path", ctypes.c_int32), ("waves", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("splits", ctypes.c_int32), ("groups_per_split", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("launches", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64),
                ("stream_k", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()


def _declare(lib):
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.quantize_rtn_int4_g128.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    lib.quantize_rtn_int4_g128.restype = i32
    lib.w4a16_packed_bytes.argtypes = [i64, i64]
    lib.w4a16_packed_bytes.restype = sz
    lib.pack_weights.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.pack_weights.restype = i32
    lib.unpack_weights.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.unpack_weights.restype = i32
    lib.w4a16_update_packed.argtypes = [vp, i64, i64, vp, i64, vp, vp, i64, i32, ctypes.c_float, ctypes.c_float,
                                        ctypes.POINTER(ctypes.c_uint64), vp]
    lib.w4a16_update_packed.restype = i32
    lib.shard_packed_weights.argtypes = [vp, i64, i64, i32, i64, i64, vp, vp]
    lib.shard_packed_weights.restype = i32
    lib.w4a16_linear_workspace_bytes.argtypes = [i64, i64, i64]
    lib.w4a16_linear_workspace_bytes.restype = sz
    lib.w4a16_linear.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.w4a16_linear.restype = i32
    lib.w4a16_linear_with_path.argtypes = [i32, vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.w4a16_linear_with_path.restype = i32
    lib.w4a16_linear_act_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.w4a16_linear_act_workspace_bytes.restype = sz
    lib.w4a16_linear_act.argtypes = [i32, i32, vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.w4a16_linear_act.restype = i32
    lib.w4a16_linear_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp]
    lib.w4a16_linear_noalloc.restype = i32
    lib.w4a16_linear_explain.argtypes = [i32, i32, i32, i64, i64, i64, ctypes.POINTER(PlanT)]
    lib.w4a16_linear_explain.restype = i32
    lib.w4a16_linear_choose_path.argtypes = [i64, i64, i64]
    lib.w4a16_linear_choose_path.restype = i32
    lib.quantize_rtn_int8_g128.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    lib.quantize_rtn_int8_g128.restype = i32
    lib.w8a16_packed_bytes.argtypes = [i64, i64]
    lib.w8a16_packed_bytes.restype = sz
    lib.pack_weights_int8.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.pack_weights_int8.restype = i32
    lib.unpack_weights_int8.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.unpack_weights_int8.restype = i32
    lib.w8a16_linear_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.w8a16_linear_workspace_bytes.restype = sz
    lib.w8a16_linear.argtypes = [i32, i32, vp, i32, i64, i64, i64, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.w8a16_linear.restype = i32
    lib.w8a16_linear_choose_path.argtypes = [i64, i64, i64]
    lib.w8a16_linear_choose_path.restype = i32
    lib.w8a16_update_packed.argtypes = [vp, i64, i64, vp, i64, vp, vp, i64, i32, ctypes.c_float, ctypes.c_float,
                                        ctypes.POINTER(ctypes.c_uint64), vp]
    lib.w8a16_update_packed.restype = i32
    lib.shard_packed_weights_int8.argtypes = [vp, i64, i64, i32, i64, i64, vp, vp]
    lib.shard_packed_weights_int8.restype = i32
    lib.w4a16_status_string.argtypes = [i32]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    return lib


def lib():
    """The loaded C library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"HIP library not built ({LIB_PATH} missing): run "
                        "`python -m weight_only_int4_rtn_amd.build`")
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    return lib().w4a16_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status == OK:
        return
    if status in (EINVAL, EUNSUPPORTED, EWORKSPACE):
        raise W4A16ArgumentError(status, what)
    raise W4A16LaunchError(status, what)


def _need(t, dtype, what: str, nbytes: int | None = None, shape=None):
    """Host-side checks of a tensor argument before any launch: dtype, shape,
    and at least ``nbytes`` bytes of storage from its data pointer."""
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if nbytes is not None:
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{what} holds {have} bytes, the layer needs {nbytes}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _act_tag(dtype) -> int:  # activation dtype tag
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float16:
        return F16
    raise ValueError(f"activations must be bfloat16 or float16, got {dtype}")


def _w_tag(dtype) -> int:
    if dtype == torch.float32:
        return F32
    return _act_tag(dtype)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")


# ---------------------------------------------------------------------------


def _bits(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError(f"weights are INT4 or INT8 (bits 4 or 8), got {bits}")
    return bits


def packed_bytes(n: int, k: int, bits: int = 4) -> int:
    if _bits(bits) == 8:
        return int(lib().w8a16_packed_bytes(n, k))
    return int(lib().w4a16_packed_bytes(n, k))


def workspace_bytes(m: int, n: int, k: int, act: Act = Act.NONE, bits: int = 4) -> int:
    if _bits(bits) == 8:
        return int(lib().w8a16_linear_workspace_bytes(int(act), m, n, k))
    if act == Act.NONE:
        return int(lib().w4a16_linear_workspace_bytes(m, n, k))
    return int(lib().w4a16_linear_act_workspace_bytes(int(act), m, n, k))


def choose_path(m: int, n: int, k: int, bits: int = 4) -> Path:
    if _bits(bits) == 8:
        return Path(lib().w8a16_linear_choose_path(m, n, k))
    return Path(lib().w4a16_linear_choose_path(m, n, k))


def explain(m: int, n: int, k: int, act: Act = Act.NONE, path: Path = Path.AUTO, bits: int = 4) -> dict:
    """The plan a linear call of these sizes runs (w4a16_linear_explain)."""
    plan = PlanT()
    _check(lib().w4a16_linear_explain(_bits(bits), int(act), int(path), m, n, k, ctypes.byref(plan)),
           "w4a16_linear_explain")
    out = {f: getattr(plan, f) for f, _ in PlanT._fields_ if f != "reserved"}
    out["path"] = Path(out["path"])
    return out


def quantize(w: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """RTN INT4 g128: w [n, k] (f32/bf16/f16, rows contiguous) -> (codes [n, k/2] uint8, scales [n, k/128] f32).
    ``codes`` and ``scales`` may be given as preallocated outputs."""
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D tensor with contiguous rows")
    n, k = w.shape
    if codes is not None:
        _need(codes, torch.uint8, "codes", shape=(n, k // 2))
    if scales is not None:
        _need(scales, torch.float32, "scales", shape=(n, k // GROUP))
    _require_cuda(w, codes, scales)
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // GROUP), dtype=torch.float32, device=w.device)
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("codes and scales must be contiguous")
    st = lib().quantize_rtn_int4_g128(_ptr(w), _w_tag(w.dtype), n, k, w.stride(0), _ptr(codes),
                                      _ptr(scales), _stream(w.device))
    _check(st, "quantize_rtn_int4_g128")
    return codes, scales


def pack(codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Canonical codes [n, k/2] + scales [n, k/128] -> packed execution layout (uint8, 1-D);
    ``out`` may be a preallocated uint8 buffer of at least packed_bytes(n, k) bytes."""
    if codes.dim() != 2:
        raise ValueError("codes must be a 2-D [n, k/2] uint8 tensor")
    n, half = codes.shape
    k = 2 * half
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float32, "scales", shape=(n, k // GROUP))
    _require_cuda(codes, scales)
    codes = codes.contiguous()
    scales = scales.contiguous()
    nbytes = packed_bytes(n, k)
    if nbytes == 0 and n > 0:
        raise ValueError(f"invalid layer shape n={n}, k={k}")
    if out is not None:
        _need(out, torch.uint8, "out", nbytes)
        _require_cuda(out)
        packed = out
    else:
        packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    st = lib().pack_weights(_ptr(codes), _ptr(scales), n, k, _ptr(packed), _stream(codes.device))
    _check(st, "pack_weights")
    return packed


def unpack(packed: torch.Tensor, n: int, k: int):
    """Packed INT4 weight -> canonical (codes [n, k/2] uint8, scales [n, k/128] f32)."""
    _need(packed, torch.uint8, "packed", packed_bytes(n, k))
    _require_cuda(packed)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((n, k // GROUP), dtype=torch.float32, device=packed.device)
    st = lib().unpack_weights(_ptr(packed), n, k, _ptr(codes), _ptr(scales), _stream(packed.device))
    _check(st, "unpack_weights")
    return codes, scales


def quantize_int8(w: torch.Tensor):
    """RTN INT8 g128: w [n, k] (f32/bf16/f16, rows contiguous) -> (codes [n, k] int8, scales [n, k/128] f32)."""
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D tensor with contiguous rows")
    _require_cuda(w)
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.int8, device=w.device)
    scales = torch.empty((n, k // GROUP), dtype=torch.float32, device=w.device)
    st = lib().quantize_rtn_int8_g128(_ptr(w), _w_tag(w.dtype), n, k, w.stride(0), _ptr(codes),
                                      _ptr(scales), _stream(w.device))
    _check(st, "quantize_rtn_int8_g128")
    return codes, scales


def pack_int8(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """INT8 codes [n, k] + scales [n, k/128] -> packed INT8 execution layout (uint8, 1-D)."""
    if codes.dtype != torch.int8 or codes.dim() != 2:
        raise ValueError("INT8 codes must be a 2-D [n, k] torch.int8 tensor")
    n, k = codes.shape
    _need(scales, torch.float32, "scales", shape=(n, k // GROUP))
    _require_cuda(codes, scales)
    codes = codes.contiguous()
    scales = scales.contiguous()
    nbytes = packed_bytes(n, k, 8)
    if nbytes == 0 and n > 0:
        raise ValueError(f"invalid layer shape n={n}, k={k}")
    packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    st = lib().pack_weights_int8(_ptr(codes), _ptr(scales), n, k, _ptr(packed), _stream(codes.device))
    _check(st, "pack_weights_int8")
    return packed


def unpack_int8(packed: torch.Tensor, n: int, k: int):
    """Packed INT8 weight -> canonical (codes [n, k] int8, scales [n, k/128] f32)."""
    _need(packed, torch.uint8, "packed", packed_bytes(n, k, 8))
    _require_cuda(packed)
    codes = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    scales = torch.empty((n, k // GROUP), dtype=torch.float32, device=packed.device)
    st = lib().unpack_weights_int8(_ptr(packed), n, k, _ptr(codes), _ptr(scales), _stream(packed.device))
    _check(st, "unpack_weights_int8")
    return codes, scales


def update_(packed: torch.Tensor, n: int, k: int, update: torch.Tensor | None = None,
            mat1: torch.Tensor | None = None, mat2: torch.Tensor | None = None,
            alpha: float = 1.0, beta: float = 1.0, seed: int | None = None, bits: int = 4) -> torch.Tensor:
    """In place: packed <- requantize(beta * dequant(packed) + alpha * U), U the
    dense ``update`` [n, k] or ``mat1`` [n, r] @ ``mat2`` [r, k]; stochastic
    rounding when ``seed`` (unsigned 64-bit) is given; ``bits=8`` for a
    packed INT8 weight."""
    bits = _bits(bits)
    _need(packed, torch.uint8, "packed", packed_bytes(n, k, bits))
    if (update is None) == (mat1 is None or mat2 is None):
        raise ValueError("pass either update, or mat1 and mat2")
    src = update if update is not None else mat1
    dt = _w_tag(src.dtype)
    rank = 0
    ldu = 0
    if update is not None:
        if update.dim() != 2 or tuple(update.shape) != (n, k) or update.stride(-1) != 1:
            raise ValueError("update must be [n, k] with unit column stride")
        ldu = update.stride(0)
    else:
        if mat1.dim() != 2 or mat2.dim() != 2:
            raise ValueError("mat1 [n, r] and mat2 [r, k] must be 2-D")
        mat1 = mat1.contiguous()
        mat2 = mat2.contiguous()
        if mat2.dtype != mat1.dtype or mat1.shape[0] != n or mat2.shape != (mat1.shape[1], k):
            raise ValueError("mat1 [n, r] and mat2 [r, k] of one dtype")
        rank = mat1.shape[1]
    _require_cuda(packed, update, mat1, mat2)
    sp = None
    if seed is not None:
        sp = ctypes.pointer(ctypes.c_uint64(int(seed) & ((1 << 64) - 1)))
    fn = lib().w8a16_update_packed if bits == 8 else lib().w4a16_update_packed
    st = fn(_ptr(packed), n, k, _ptr(update), ldu, _ptr(mat1), _ptr(mat2), rank, dt,
            float(alpha), float(beta), sp, _stream(packed.device))
    _check(st, "w8a16_update_packed" if bits == 8 else "w4a16_update_packed")
    return packed


def shard(packed: torch.Tensor, n: int, k: int, dim: int, start: int, length: int, bits: int = 4) -> torch.Tensor:
    """Rows [start, start+length) (dim 0) or group-aligned columns (dim 1) of a
    packed [n, k] weight (INT4, or INT8 with bits=8) as a new packed weight
    (no requantization)."""
    bits = _bits(bits)
    _need(packed, torch.uint8, "packed", packed_bytes(n, k, bits))
    _require_cuda(packed)
    rows, cols = (length, k) if dim == 0 else (n, length)
    size = packed_bytes(rows, cols, bits)
    out = torch.empty(max(size, 16), dtype=torch.uint8, device=packed.device)
    fn = lib().shard_packed_weights_int8 if bits == 8 else lib().shard_packed_weights
    st = fn(_ptr(packed), n, k, dim, start, length, _ptr(out), _stream(packed.device))
    _check(st, "shard_packed_weights_int8" if bits == 8 else "shard_packed_weights")
    return out[:size]


_workspaces: dict = {}


def workspace_for(device, stream_handle: int, nbytes: int) -> torch.Tensor | None:
    """A workspace of at least ``nbytes`` for one (device, stream), zero-filled
    when allocated (the calls leave its counter header zero)."""
    if nbytes == 0:
        return None
    key = (torch.device(device).index, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def linear(x: torch.Tensor, packed: torch.Tensor, n: int, bias: torch.Tensor | None = None,
           out: torch.Tensor | None = None, path: Path = Path.AUTO,
           workspace: torch.Tensor | None = None, act: Act = Act.NONE, bits: int = 4) -> torch.Tensor:
    """y = act(x) . dequant(packed)^T + bias for x [..., k] (bf16/f16) -> y [..., n]
    (x's dtype).  With ``act=Act.SWIGLU`` the rows of x are [up | gate], 2k values.
    ``bits=8``: ``packed`` is a packed INT8 weight (``pack_int8``)."""
    bits = _bits(bits)
    if x.requires_grad or (bias is not None and bias.requires_grad):
        raise ValueError("inference only: autograd inputs are not supported")
    act = Act(act)
    dt = _act_tag(x.dtype)
    width = x.shape[-1]
    if act == Act.SWIGLU and width % 2 != 0:
        raise ValueError("SwiGLU input rows hold [up | gate]: an even number of columns")
    k = width // 2 if act == Act.SWIGLU else width
    lead = x.shape[:-1]
    x2 = x.reshape(-1, width)
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    m = x2.shape[0]
    if bias is not None:
        if bias.dtype != x.dtype or bias.shape != (n,):
            raise ValueError("bias must have shape [n] and x's dtype")
        bias = bias.contiguous()
    if out is not None:
        if out.shape != (*lead, n) or out.dtype != x.dtype:
            raise ValueError("out must have shape [..., n] and x's dtype")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    _need(packed, torch.uint8, "packed", packed_bytes(n, k, bits))
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    need = workspace_bytes(m, n, k, act, bits)
    if Path(path) == Path.GEMM_STREAMK and m > 0 and n > 0:
        need = max(need, explain(m, n, k, act, path, bits)["workspace_bytes"])
    if workspace is None and need > 0 and torch.cuda.is_current_stream_capturing():
        # a workspace allocated here would belong to the graph's memory pool
        # and its zero fill would only run at replay: a captured call needs
        # its own workspace, zero-filled before the capture
        raise ValueError(f"this call needs a {need}-byte workspace: under graph capture pass a "
                         "zero-filled workspace= allocated before the capture")
    _require_cuda(x, packed, bias, out, workspace)
    if out is None:
        out = torch.empty((*lead, n), dtype=x.dtype, device=x.device)
    y2 = out.view(-1, n)
    stream = _stream(x.device)
    if workspace is None:
        workspace = workspace_for(x.device, stream.value, need)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if bits == 8:
        st = lib().w8a16_linear(int(act), int(path), _ptr(x2), dt, m, k, x2.stride(0), _ptr(packed), n,
                                _ptr(bias), _ptr(y2), n, _ptr(workspace), ws_bytes, stream)
        _check(st, "w8a16_linear")
        return out
    if act == Act.NONE:
        st = lib().w4a16_linear_with_path(int(path), _ptr(x2), dt, m, k, x2.stride(0), _ptr(packed), n,
                                          _ptr(bias), _ptr(y2), n, _ptr(workspace), ws_bytes, stream)
    else:
        st = lib().w4a16_linear_act(int(act), int(path), _ptr(x2), dt, m, k, x2.stride(0), _ptr(packed), n,
                                    _ptr(bias), _ptr(y2), n, _ptr(workspace), ws_bytes, stream)
    _check(st, "w4a16_linear_act" if act != Act.NONE else "w4a16_linear")
    return out


def linear_noalloc(x: torch.Tensor, packed: torch.Tensor, n: int, bias: torch.Tensor | None = None,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """y = x . dequant(packed)^T + bias through w4a16_linear_noalloc: the
    library's fixed per-GPU scratch array stands in for the workspace, so the
    call allocates nothing (pass ``out`` to allocate nothing here either).
    Calls that may overlap on one GPU race on that array."""
    dt = _act_tag(x.dtype)
    k = x.shape[-1]
    lead = x.shape[:-1]
    x2 = x.reshape(-1, k)
    if x2.stride(-1) != 1:
        raise ValueError("x rows must be contiguous")
    m = x2.shape[0]
    if bias is not None and (bias.dtype != x.dtype or bias.shape != (n,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [n] tensor of x's dtype")
    if out is not None and (out.shape != (*lead, n) or out.dtype != x.dtype or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [..., n] tensor of x's dtype")
    _need(packed, torch.uint8, "packed", packed_bytes(n, k))
    _require_cuda(x, packed, bias, out)
    if out is None:
        out = torch.empty((*lead, n), dtype=x.dtype, device=x.device)
    st = lib().w4a16_linear_noalloc(_ptr(x2), dt, m, k, x2.stride(0), _ptr(packed), n, _ptr(bias),
                                    _ptr(out.view(-1, n)), n, _stream(x.device))
    _check(st, "w4a16_linear_noalloc")
    return out
