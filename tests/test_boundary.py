"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments from host metadata alone (no GPU needed: every check here
returns before anything is launched).

The validation contract: arguments are checked from shapes, dtypes,
alignment and sizes only, never from tensor contents ("Piper Kernels",
section "Validation contract")."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

import weight_only_int4_rtn_amd as w4  # noqa: E402
from weight_only_int4_rtn_amd import _binding as B  # noqa: E402

A = 1 << 20  # a 16-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    return w4.lib()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"quantize_rtn_int4_g128", "pack_weights", "w4a16_linear", "unpack_weights",
            "w4a16_packed_bytes", "w4a16_linear_workspace_bytes", "w4a16_status_string",
            "w4a16_linear_with_path", "w4a16_linear_choose_path", "w4a16_linear_act",
            "w4a16_linear_act_workspace_bytes", "shard_packed_weights", "w4a16_update_packed",
            "quantize_rtn_int8_g128", "w8a16_packed_bytes", "pack_weights_int8", "unpack_weights_int8",
            "w8a16_linear_workspace_bytes", "w8a16_linear", "w8a16_linear_choose_path",
            "shard_packed_weights_int8", "w8a16_update_packed"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_single_hip_runtime_loaded(lib):
    maps = open("/proc/self/maps").read()
    runtimes = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(runtimes) == 1, runtimes


def test_status_strings(lib):
    for s in range(5):
        assert w4.status_string(s)
    assert w4.status_string(99) == "unknown status"


def test_packed_bytes(lib):
    # 16-row tiles x 128-column groups, 1024 code bytes + 64 scale bytes each
    assert w4.packed_bytes(16, 128) == 1088
    assert w4.packed_bytes(17, 256) == 2 * 2 * 1088
    assert w4.packed_bytes(32768, 2048) == 2048 * 16 * 1088
    assert w4.packed_bytes(0, 128) == 0
    assert w4.packed_bytes(16, 100) == 0
    assert w4.packed_bytes(16, 0) == 0
    assert w4.packed_bytes(-1, 128) == 0


def test_choose_path(lib):
    assert w4.choose_path(1, 2048, 2048) == w4.Path.GEMV
    for m in (1, 2, 3, 4, 8, 16, 50, 64, 256, 1024, 4096):
        assert w4.choose_path(m, 2048, 2048) != w4.Path.AUTO
    assert w4.choose_path(4096, 2048, 2048) == w4.Path.GEMM
    # measured crossovers: MFMA small-M kernel up to M = 8 on <= 16384 outputs,
    # the mid-M kernel up to M = 96 on layers above 8 M weights
    assert w4.choose_path(2, 2560, 2048) == w4.Path.GEMV
    assert w4.choose_path(2, 32768, 2048) == w4.Path.MGEMV
    assert w4.choose_path(2, 1024, 4096) == w4.Path.MGEMV
    # the mid-M kernel from M = 3 where it needs no K split (>= 16384 outputs,
    # K <= 2048) and where the small-M kernel's split would need the reduce
    # launch; the small-M kernel keeps M = 2 and the other split layers
    assert w4.choose_path(8, 16384, 2048) == w4.Path.SKINNY
    assert w4.choose_path(3, 32768, 2048) == w4.Path.SKINNY
    assert w4.choose_path(2, 16384, 2048) == w4.Path.MGEMV
    assert w4.choose_path(8, 4096, 16384) == w4.Path.SKINNY
    assert w4.choose_path(4, 2048, 16384) == w4.Path.MGEMV
    assert w4.choose_path(8, 2048, 16384) == w4.Path.MGEMV
    assert w4.choose_path(8, 16384, 4096) == w4.Path.SKINNY
    assert w4.choose_path(6, 2048, 16384) == w4.Path.MGEMV
    assert w4.choose_path(4, 16384, 4096) == w4.Path.MGEMV
    assert w4.choose_path(16, 2560, 2048) == w4.Path.MGEMV
    assert w4.choose_path(8, 32768, 2048) == w4.Path.SKINNY
    assert w4.choose_path(64, 32768, 2048) == w4.Path.SKINNY
    assert w4.choose_path(65, 32768, 2048) == w4.Path.GEMM
    assert w4.choose_path(128, 16384, 2048) == w4.Path.SKINNY
    assert w4.choose_path(128, 2048, 16384) == w4.Path.SKINNY
    assert w4.choose_path(129, 16384, 2048) == w4.Path.GEMM
    assert w4.choose_path(512, 4096, 1024) == w4.Path.SKINNY
    assert w4.choose_path(513, 4096, 1024) == w4.Path.GEMM


def test_workspace_bytes(lib):
    assert w4.workspace_bytes(0, 2048, 2048) == 0
    assert w4.workspace_bytes(1, 2048, 100) == 0
    # a long-K decode shape splits K across workgroups and needs a workspace
    assert w4.workspace_bytes(1, 2048, 16384) > 0


def q(lib, w, dt, n, k, ldw, codes, scales):
    return lib.quantize_rtn_int4_g128(w, dt, n, k, ldw, codes, scales, None)


def test_quantize_rejects(lib):
    assert q(lib, A, B.F32, 4, 100, 100, A * 2, A * 3) == B.EINVAL      # k % 128
    assert q(lib, A, B.F32, 4, 0, 128, A * 2, A * 3) == B.EINVAL        # k == 0
    assert q(lib, A, B.F32, -1, 128, 128, A * 2, A * 3) == B.EINVAL     # n < 0
    assert q(lib, A, B.F32, 4, 256, 128, A * 2, A * 3) == B.EINVAL      # ldw < k
    assert q(lib, A, 7, 4, 128, 128, A * 2, A * 3) == B.EUNSUPPORTED    # dtype
    assert q(lib, None, B.F32, 4, 128, 128, A * 2, A * 3) == B.EINVAL   # null
    assert q(lib, A, B.F32, 4, 128, 128, None, A * 3) == B.EINVAL
    assert q(lib, A + 4, B.F32, 4, 128, 128, A * 2, A * 3) == B.EINVAL  # misaligned w
    assert q(lib, A, B.F32, 4, 128, 130, A * 2, A * 3) == B.EINVAL      # row stride not 16 B
    assert q(lib, A, B.F32, 4, 128, 128, A * 2 + 1, A * 3) == B.EINVAL  # misaligned codes
    assert q(lib, A, B.F32, 4, 128, 128, A, A * 3) == B.EINVAL          # codes overlap w
    assert q(lib, A, B.F32, 0, 128, 128, None, None) == B.OK            # empty: no-op


def test_pack_rejects(lib):
    assert lib.pack_weights(A, A * 2, 4, 100, A * 3, None) == B.EINVAL
    assert lib.pack_weights(None, A * 2, 4, 128, A * 3, None) == B.EINVAL
    assert lib.pack_weights(A, A * 2, 4, 128, A * 3 + 8, None) == B.EINVAL
    assert lib.pack_weights(A, A * 2, 4, 128, A, None) == B.EINVAL       # packed overlaps codes
    assert lib.pack_weights(A, A * 2, 0, 128, A * 3, None) == B.OK
    assert lib.unpack_weights(A * 3, 4, 100, A, A * 2, None) == B.EINVAL
    assert lib.unpack_weights(A * 3, 4, 128, A, A, None) == B.EINVAL      # codes overlap scales
    assert lib.unpack_weights(A * 3, 0, 128, A, A * 2, None) == B.OK


def lin(lib, x=A, act=B.BF16, m=1, k=128, ldx=128, packed=A * 4, n=16, bias=None, y=A * 8, ldy=16,
        ws=None, ws_bytes=0, path=0):
    return lib.w4a16_linear_with_path(path, x, act, m, k, ldx, packed, n, bias, y, ldy, ws, ws_bytes, None)


def test_linear_rejects(lib):
    assert lin(lib, k=100, ldx=104) == B.EINVAL                   # k % 128
    assert lin(lib, act=B.F32) == B.EUNSUPPORTED                  # activation dtype
    assert lin(lib, ldx=64) == B.EINVAL                           # ldx < k
    assert lin(lib, k=128, ldx=130) == B.EINVAL                   # ldx % 8
    assert lin(lib, ldy=8) == B.EINVAL                            # ldy < n
    assert lin(lib, m=-1) == B.EINVAL
    assert lin(lib, x=None) == B.EINVAL
    assert lin(lib, packed=None) == B.EINVAL
    assert lin(lib, y=None) == B.EINVAL
    assert lin(lib, x=A + 2) == B.EINVAL                          # misaligned x
    assert lin(lib, y=A + 1) == B.EINVAL                          # misaligned y
    assert lin(lib, y=A) == B.EINVAL                              # y overlaps x
    assert lin(lib, y=A * 4) == B.EINVAL                          # y overlaps packed
    assert lin(lib, path=9) == B.EINVAL                           # unknown path
    assert lin(lib, m=0) == B.OK                                  # empty: no-op
    assert lin(lib, n=0, ldy=0) == B.OK
    # a K beyond one workgroup's reach (32 groups) splits and needs a workspace
    gemv = int(w4.Path.GEMV)
    need = w4.workspace_bytes(1, 2048, 32768)
    assert lin(lib, m=1, k=32768, ldx=32768, n=2048, ldy=2048, y=A * 64, path=gemv) == B.EWORKSPACE
    assert need > 256
    assert lin(lib, m=1, k=32768, ldx=32768, n=2048, ldy=2048, y=A * 64, ws=A * 128,
               ws_bytes=256, path=gemv) == B.EWORKSPACE
    assert lin(lib, m=1, k=32768, ldx=32768, n=2048, ldy=2048, y=A * 64, ws=A * 128 + 8,
               ws_bytes=need, path=gemv) == B.EINVAL          # misaligned workspace
    # the GEMM path takes row strides up to 2^22 elements (32-bit tile offsets)
    big = (1 << 22) + 8
    assert lin(lib, m=256, k=128, ldx=big, n=16, y=A * 4096, path=int(w4.Path.GEMM)) == B.EUNSUPPORTED
    assert w4.choose_path(256, 16, (1 << 22) + 128) == w4.Path.SKINNY


def lin_act(lib, fn, path=0, x=A, act=B.BF16, m=1, k=128, ldx=256, packed=A * 4, n=16, bias=None, y=A * 8,
            ldy=16, ws=None, ws_bytes=0):
    return lib.w4a16_linear_act(fn, path, x, act, m, k, ldx, packed, n, bias, y, ldy, ws, ws_bytes, None)


def test_linear_act_rejects(lib):
    sw, ge = int(w4.Act.SWIGLU), int(w4.Act.GELU_TANH)
    assert lin_act(lib, 3) == B.EINVAL                             # unknown activation
    assert lin_act(lib, -1) == B.EINVAL
    assert lin_act(lib, sw, ldx=128) == B.EINVAL                   # [up | gate] needs ldx >= 2k
    assert lin_act(lib, ge, ldx=120) == B.EINVAL                   # ldx < k
    assert lin_act(lib, sw, act=B.F32) == B.EUNSUPPORTED
    assert lin_act(lib, sw, path=9) == B.EINVAL
    # y inside the gate half of x's row span overlaps x
    assert lin_act(lib, sw, m=2, y=A + 2 * 200) == B.EINVAL
    assert lin_act(lib, sw, m=0) == B.OK                            # empty: no-op
    assert lin_act(lib, sw, n=0, ldy=0) == B.OK
    # the large-M path materialises the activated input in the workspace
    gemm = int(w4.Path.GEMM)
    need = w4.workspace_bytes(256, 16, 128, w4.Act.SWIGLU)
    assert need >= 256 * 128 * 2
    assert w4.workspace_bytes(256, 16, 128) == 0
    assert lin_act(lib, sw, path=gemm, m=256, y=A * 16) == B.EWORKSPACE
    assert lin_act(lib, sw, path=gemm, m=256, y=A * 16, ws=A * 32, ws_bytes=need - 16) == B.EWORKSPACE
    assert lin_act(lib, sw, path=gemm, m=256, y=A * 16, ws=A, ws_bytes=need) == B.EINVAL  # workspace overlaps x
    # with an activation the GEMM's row-stride limit applies to k, not ldx
    big = (1 << 22) + 8
    assert lin_act(lib, ge, path=gemm, m=256, k=(1 << 22) + 128, ldx=(1 << 22) + 128, n=16,
                   y=A * 8192) == B.EUNSUPPORTED
    assert lin_act(lib, ge, path=gemm, m=256, k=128, ldx=big, y=A * 8192, ws=None) == B.EWORKSPACE
    # an unsplit GEMM keeps the activated input after the 1 MiB header of
    # exchange slots, never inside it
    assert w4.workspace_bytes(300, 4104, 640) == 0
    assert w4.workspace_bytes(300, 4104, 640, w4.Act.GELU_TANH) >= (1 << 20) + 300 * 640 * 2
    assert lib.w4a16_linear_act_workspace_bytes(5, 16, 16, 128) == 0
    assert lib.w4a16_linear_act_workspace_bytes(int(w4.Act.NONE), 1, 2048, 16384) == w4.workspace_bytes(1, 2048, 16384)


def test_update_rejects(lib):
    import ctypes
    up = lib.w4a16_update_packed
    seed = ctypes.pointer(ctypes.c_uint64(5))
    f1 = ctypes.c_float(1.0)
    assert up(A, 16, 128, A * 4, 128, None, None, 0, 7, f1, f1, None, None) == B.EUNSUPPORTED   # dtype
    assert up(A, 16, 100, A * 4, 128, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL     # k % 128
    assert up(A, 16, 128, None, 0, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL        # no update
    assert up(A, 16, 128, A * 4, 128, A * 8, A * 9, 4, B.F32, f1, f1, None, None) == B.EINVAL   # both forms
    assert up(A, 16, 128, None, 0, A * 8, None, 4, B.F32, f1, f1, None, None) == B.EINVAL       # mat2 missing
    assert up(A, 16, 128, None, 0, A * 8, A * 9, 0, B.F32, f1, f1, None, None) == B.EINVAL      # rank 0 low-rank
    assert up(A, 16, 128, None, 0, A * 8, A * 9, (1 << 16) + 1, B.F32, f1, f1, seed, None) == B.EINVAL  # rank
    assert up(A, 16, 128, A * 4, 120, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL     # ldu < k
    assert up(A, 16, 128, A * 4, 130, None, None, 0, B.BF16, f1, f1, None, None) == B.EINVAL    # ldu bytes % 16
    assert up(A, 16, 128, A * 4 + 8, 128, None, None, 0, B.BF16, f1, f1, None, None) == B.EINVAL  # alignment
    assert up(A, 16, 128, A + 64, 128, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL    # overlaps packed
    assert up(None, 16, 128, A * 4, 128, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL
    assert up(A, 0, 128, A * 4, 128, None, None, 0, B.F32, f1, f1, seed, None) == B.OK          # empty: no-op


def test_shard_rejects(lib):
    sh = lib.shard_packed_weights
    assert sh(A, 100, 640, 2, 0, 10, A * 4, None) == B.EINVAL        # dim
    assert sh(A, 100, 640, 0, -1, 10, A * 4, None) == B.EINVAL       # start < 0
    assert sh(A, 100, 640, 0, 0, 0, A * 4, None) == B.EINVAL         # empty shard
    assert sh(A, 100, 640, 0, 95, 10, A * 4, None) == B.EINVAL       # past n
    assert sh(A, 100, 640, 1, 64, 128, A * 4, None) == B.EINVAL      # start not on a group
    assert sh(A, 100, 640, 1, 128, 100, A * 4, None) == B.EINVAL     # length not whole groups
    assert sh(A, 100, 640, 1, 512, 256, A * 4, None) == B.EINVAL     # past k
    assert sh(A, 100, 600, 0, 0, 10, A * 4, None) == B.EINVAL        # k % 128
    assert sh(A, 0, 640, 0, 0, 1, A * 4, None) == B.EINVAL           # empty weight
    assert sh(None, 100, 640, 0, 0, 10, A * 4, None) == B.EINVAL
    assert sh(A, 100, 640, 0, 0, 10, A + 8, None) == B.EINVAL        # misaligned / overlapping out
    assert sh(A, 100, 640, 0, 0, 10, A + 4096, None) == B.EINVAL     # out inside the packed weight


def test_int8_packed_bytes_and_paths(lib):
    # 16-row tiles x 128-column groups, 2048 code bytes + 64 scale bytes each
    assert w4.packed_bytes(16, 128, bits=8) == 2112
    assert w4.packed_bytes(17, 256, bits=8) == 2 * 2 * 2112
    assert w4.packed_bytes(0, 128, bits=8) == 0
    assert w4.packed_bytes(16, 100, bits=8) == 0
    with pytest.raises(ValueError):
        w4.packed_bytes(16, 128, bits=2)
    assert w4.choose_path(1, 2048, 2048, bits=8) == w4.Path.GEMV
    assert w4.choose_path(2, 2048, 2048, bits=8) == w4.Path.GEMV
    assert w4.choose_path(2, 32768, 2048, bits=8) == w4.Path.MGEMV
    for m in (3, 4, 8, 16):
        assert w4.choose_path(m, 2048, 2048, bits=8) == w4.Path.MGEMV
    assert w4.choose_path(8, 16384, 2048, bits=8) == w4.Path.MGEMV
    assert w4.choose_path(9, 16384, 2048, bits=8) == w4.Path.SKINNY
    for m in (17, 50, 127, 512):
        assert w4.choose_path(m, 2048, 2048, bits=8) == w4.Path.SKINNY
    for m in (513, 4096):
        assert w4.choose_path(m, 2048, 2048, bits=8) == w4.Path.GEMM
    assert w4.choose_path(64, 2048, 16384, bits=8) == w4.Path.SKINNY
    assert w4.choose_path(65, 2048, 16384, bits=8) == w4.Path.GEMM
    assert w4.choose_path(256, 16, (1 << 22) + 128, bits=8) == w4.Path.SKINNY
    assert w4.workspace_bytes(1, 2048, 100, bits=8) == 0
    assert w4.workspace_bytes(1, 2048, 16384, bits=8) > 0
    assert lib.w8a16_linear_workspace_bytes(5, 16, 16, 128) == 0       # unknown activation


def test_int8_quantize_and_pack_reject(lib):
    q8 = lib.quantize_rtn_int8_g128
    assert q8(A, B.F32, 4, 100, 100, A * 2, A * 3, None) == B.EINVAL      # k % 128
    assert q8(A, 7, 4, 128, 128, A * 2, A * 3, None) == B.EUNSUPPORTED    # dtype
    assert q8(A, B.F32, 4, 128, 128, A * 2 + 4, A * 3, None) == B.EINVAL  # codes not 8-byte aligned
    assert q8(A, B.F32, 4, 128, 128, A, A * 3, None) == B.EINVAL          # codes overlap w
    assert q8(A, B.F32, 4, 128, 128, A * 2, A * 2 + 256, None) == B.EINVAL  # scales inside the codes
    assert q8(A, B.F32, 0, 128, 128, None, None, None) == B.OK            # empty: no-op
    assert lib.pack_weights_int8(A, A * 2, 4, 100, A * 3, None) == B.EINVAL
    assert lib.pack_weights_int8(A, A * 2, 4, 128, A * 3 + 8, None) == B.EINVAL
    assert lib.pack_weights_int8(A, A * 2, 4, 128, A + 256, None) == B.EINVAL  # packed overlaps codes
    assert lib.pack_weights_int8(A, A * 2, 0, 128, A * 3, None) == B.OK
    assert lib.unpack_weights_int8(A * 3, 4, 128, A, A + 256, None) == B.EINVAL  # codes overlap scales
    assert lib.unpack_weights_int8(A * 3, 0, 128, A, A * 2, None) == B.OK


def lin8(lib, fn=0, path=0, x=A, act=B.BF16, m=1, k=128, ldx=128, packed=A * 4, n=16, bias=None, y=A * 8,
         ldy=16, ws=None, ws_bytes=0):
    return lib.w8a16_linear(fn, path, x, act, m, k, ldx, packed, n, bias, y, ldy, ws, ws_bytes, None)


def test_int8_linear_rejects(lib):
    assert lin8(lib, 3) == B.EINVAL                                         # unknown activation
    big = (1 << 22) + 8
    assert lin8(lib, path=int(w4.Path.GEMM), m=256, ldx=big, y=A * 4096) == B.EUNSUPPORTED  # 32-bit x offsets
    assert lin8(lib, path=9) == B.EINVAL
    assert lin8(lib, act=B.F32) == B.EUNSUPPORTED
    assert lin8(lib, k=100, ldx=104) == B.EINVAL
    assert lin8(lib, fn=int(w4.Act.SWIGLU), ldx=128) == B.EINVAL             # [up | gate] needs 2k
    assert lin8(lib, y=A * 4 + 2048) == B.EINVAL                            # y inside the INT8 packed weight
    assert lin8(lib, y=A * 4 + 1200) == B.EINVAL                            # (an INT4 weight would end at 1088)
    assert lin8(lib, m=0) == B.OK
    need = w4.workspace_bytes(1, 2048, 32768, bits=8)
    assert need > 0
    assert lin8(lib, m=1, k=32768, ldx=32768, n=2048, ldy=2048, y=A * 1024, path=int(w4.Path.GEMV)) == B.EWORKSPACE


def test_int8_update_rejects(lib):
    import ctypes
    up = lib.w8a16_update_packed
    f1 = ctypes.c_float(1.0)
    assert up(A, 16, 128, A * 4, 128, None, None, 0, 7, f1, f1, None, None) == B.EUNSUPPORTED   # dtype
    assert up(A, 16, 128, None, 0, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL        # no update
    assert up(A, 16, 128, A * 4, 120, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL     # ldu < k
    # the update inside the INT8 packed weight (2112 bytes; an INT4 one ends at 1088)
    assert up(A, 16, 128, A + 1536, 128, None, None, 0, B.F32, f1, f1, None, None) == B.EINVAL
    assert up(A, 0, 128, A * 4, 128, None, None, 0, B.F32, f1, f1, None, None) == B.OK          # empty: no-op


def test_int8_shard_rejects(lib):
    sh = lib.shard_packed_weights_int8
    assert sh(A, 100, 640, 2, 0, 10, A * 4, None) == B.EINVAL        # dim
    assert sh(A, 100, 640, 0, 95, 10, A * 4, None) == B.EINVAL       # past n
    assert sh(A, 100, 640, 1, 64, 128, A * 4, None) == B.EINVAL      # start not on a group
    assert sh(A, 0, 640, 0, 0, 1, A * 4, None) == B.EINVAL           # empty weight
    # an INT8 weight of 100 x 640 spans 7 tiles x 5 groups x 2112 bytes: an
    # output 40 KB in overlaps it (an INT4 weight ends at 38080 bytes)
    assert w4.packed_bytes(100, 640, bits=8) == 7 * 5 * 2112
    assert sh(A, 100, 640, 0, 0, 10, A + 40960, None) == B.EINVAL


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        w4.quantize(torch.zeros(16, 128))


def test_status_maps_to_exception_type(lib):
    # EINVAL, EUNSUPPORTED and EWORKSPACE reject a request from its
    # arguments: ValueError; EHIP is a runtime failure: RuntimeError
    for status in (B.EINVAL, B.EUNSUPPORTED, B.EWORKSPACE):
        with pytest.raises(ValueError) as ei:
            B._check(status, "call")
        assert ei.value.status == status and not isinstance(ei.value, RuntimeError)
        assert isinstance(ei.value, w4.W4A16Error)
    with pytest.raises(RuntimeError) as ei:
        B._check(B.EHIP, "call")
    assert ei.value.status == B.EHIP and not isinstance(ei.value, ValueError)
    B._check(B.OK, "call")  # no exception


def test_binding_checks_tensor_sizes_before_any_launch(lib):
    """Every size, dtype and shape mismatch between a tensor and the (n, k,
    bits) passed with it is rejected on the host, before the device check and
    before any launch (so these run without a GPU, on CPU tensors)."""
    import torch
    n, k = 40, 256
    p4 = torch.zeros(w4.packed_bytes(n, k), dtype=torch.uint8)
    x = torch.zeros(3, k, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="packed holds"):
        w4.linear(x, p4[:-64], n)                            # packed too small for (n, k)
    with pytest.raises(ValueError, match="packed holds"):
        w4.linear(x, p4, n + 16)                             # n larger than the packed weight
    with pytest.raises(ValueError, match="packed holds"):
        w4.linear(x, p4, n, bits=8)                          # an INT4 weight passed as INT8
    with pytest.raises(ValueError, match="packed must be torch.uint8"):
        w4.linear(x, p4.view(torch.int8), n)
    with pytest.raises(ValueError, match="bias"):
        w4.linear(x, p4, n, torch.zeros(n, dtype=torch.float16))
    with pytest.raises(ValueError, match="out must"):
        w4.linear(x, p4, n, out=torch.zeros(3, n + 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="contiguous"):
        w4.linear(x, p4, n, out=torch.zeros(n, 3, dtype=torch.bfloat16).t())
    with pytest.raises(ValueError, match="on a GPU"):
        w4.linear(x, p4, n)                                  # everything matches: only the device is wrong
    codes = torch.zeros(n, k // 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales must be torch.float32"):
        w4.pack(codes, torch.zeros(n, k // 128, dtype=torch.float16))
    with pytest.raises(ValueError, match="scales must have shape"):
        w4.pack(codes, torch.zeros(n, k // 128 + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="codes must be torch.uint8"):
        w4.pack(codes.view(torch.int8), torch.zeros(n, k // 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="scales must have shape"):
        w4.pack_int8(torch.zeros(n, k, dtype=torch.int8), torch.zeros(n + 1, k // 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="packed holds"):
        w4.unpack(p4[:100], n, k)
    with pytest.raises(ValueError, match="packed holds"):
        w4.unpack_int8(p4, n, k)                             # INT4-sized buffer read as INT8
    with pytest.raises(ValueError, match="packed holds"):
        w4.shard(p4[:1000], n, k, 0, 0, 16)
    with pytest.raises(ValueError, match="packed holds"):
        w4.update_(p4[:1000], n, k, update=torch.zeros(n, k))
    with pytest.raises(ValueError, match="update must be"):
        w4.update_(p4, n, k, update=torch.zeros(n + 1, k))   # in place: a wrong n would write past packed
    with pytest.raises(ValueError, match="mat1"):
        w4.update_(p4, n, k, mat1=torch.zeros(n + 1, 4), mat2=torch.zeros(4, k))
    with pytest.raises(ValueError, match="either update"):
        w4.update_(p4, n, k)


def test_captured_call_needs_an_explicit_workspace(lib, monkeypatch):
    """Under graph capture a call whose plan needs a workspace must be given
    one (allocated and zero-filled before the capture); calls that need none
    are unaffected.  Checked from metadata before anything else."""
    import torch
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    n, k = 2048, 16384          # M = 1, K split across workgroups: needs a workspace
    assert w4.workspace_bytes(1, n, k) > 0
    p = torch.zeros(w4.packed_bytes(n, k), dtype=torch.uint8)
    x = torch.zeros(1, k, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="graph capture"):
        w4.linear(x, p, n)
    with pytest.raises(ValueError, match="on a GPU"):       # explicit workspace: past the capture rule
        w4.linear(x, p, n, workspace=torch.zeros(w4.workspace_bytes(1, n, k), dtype=torch.uint8))
    n2, k2 = 4096, 256          # two groups: no path splits K, no workspace needed
    assert w4.workspace_bytes(1, n2, k2) == 0
    with pytest.raises(ValueError, match="on a GPU"):
        w4.linear(torch.zeros(1, k2, dtype=torch.bfloat16), torch.zeros(w4.packed_bytes(n2, k2), dtype=torch.uint8), n2)


def test_noalloc_scratch_size_matches_header(lib):
    text = open(HEADER).read()
    m = re.search(r"#define W4A16_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "W4A16_NOALLOC_SCRATCH_BYTES not found"
    assert B.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    # the no-alloc call's host checks come before any device work
    import torch
    with pytest.raises(ValueError, match="packed holds"):
        w4.linear_noalloc(torch.zeros(1, 256, dtype=torch.bfloat16), torch.zeros(100, dtype=torch.uint8), 16)


def test_explain_reports_the_plan(lib):
    p = w4.explain(1, 32768, 2048)
    assert p["path"] == w4.Path.GEMV and p["tile_n"] == 16 and p["splits"] == 1 and p["launches"] == 1
    assert p["workgroups"] == 2048 and p["workspace_bytes"] == 0
    p = w4.explain(1, 2048, 16384)          # K split over workgroups: exchange slots in the workspace
    assert (p["waves"], p["splits"], p["groups_per_split"]) == (8, 2, 64) and p["workspace_bytes"] > 0
    assert p["workspace_bytes"] <= w4.workspace_bytes(1, 2048, 16384)
    p = w4.explain(1, 4096, 16384)          # 256 row tiles: unsplit, 16 chunks per wave
    assert (p["waves"], p["splits"], p["groups_per_split"], p["workgroups"]) == (8, 1, 128, 256)
    p = w4.explain(4, 2048, 16384, path=w4.Path.GEMV)  # whole tiles, 8 waves, 4 splits
    assert (p["tile_n"], p["waves"], p["splits"]) == (16, 8, 4)
    p = w4.explain(6, 1024, 2048)           # MGEMV: one launch per 16-row block
    assert p["path"] == w4.Path.MGEMV and p["tile_m"] == 6
    # small-M MFMA plans: x with the chunks (M > 4) in splits of up to 64
    # groups; towards 256 workgroups below 128 row tiles; x staged in LDS at
    # M <= 4 on larger layers, and with a fused activation up to M = 8
    p = w4.explain(8, 2048, 16384, path=w4.Path.MGEMV)
    assert (p["waves"], p["splits"], p["groups_per_split"], p["workgroups"]) == (8, 2, 64, 256)
    p = w4.explain(16, 1024, 4096, path=w4.Path.MGEMV)
    assert (p["waves"], p["splits"], p["groups_per_split"], p["workgroups"]) == (4, 4, 8, 256)
    p = w4.explain(4, 2048, 16384, path=w4.Path.MGEMV)
    assert (p["waves"], p["splits"], p["groups_per_split"]) == (8, 4, 32)
    p = w4.explain(6, 2048, 16384, path=w4.Path.MGEMV, act=w4.Act.SWIGLU)
    assert (p["waves"], p["splits"], p["groups_per_split"]) == (8, 7, 21)  # x slice <= 2048 columns x 16 rows
    # INT8 GEMV at M = 1: splits of up to 64 groups on 8 waves
    p = w4.explain(1, 2048, 16384, bits=8)
    assert (p["path"], p["waves"], p["splits"], p["groups_per_split"]) == (w4.Path.GEMV, 8, 2, 64)
    # mid-M plans on INT4 layers of <= 8 M weights: at most 8 groups per split
    p = w4.explain(128, 1024, 4096, path=w4.Path.SKINNY)
    assert (p["splits"], p["groups_per_split"], p["workgroups"]) == (4, 8, 512)
    p = w4.explain(16, 1024, 4096, path=w4.Path.SKINNY)
    assert (p["splits"], p["groups_per_split"]) == (8, 4)
    assert w4.explain(40, 1024, 2048, path=w4.Path.GEMV)["launches"] >= 10
    p = w4.explain(300, 2056, 1152, act=w4.Act.GELU_TANH, path=w4.Path.GEMM)
    assert p["launches"] == (3 if p["splits"] > 1 else 2)  # activation, GEMM (+ reduce)
    assert p["workspace_bytes"] >= 300 * 1152 * 2
    assert w4.explain(0, 2048, 2048)["launches"] == 0
    # the planner's K splits go through the reduce kernel
    p = w4.explain(1024, 2048, 16384)
    assert (p["stream_k"], p["splits"], p["launches"], p["workgroups"]) == (0, 4, 2, 256)
    # the stream-K path: runs of equal length over tiles x groups, one per
    # CU, its own workspace (not part of workspace_bytes' paths)
    p = w4.explain(1024, 2560, 2048, path=w4.Path.GEMM_STREAMK)
    assert p["path"] == w4.Path.GEMM_STREAMK and p["stream_k"] == 1 and p["workgroups"] == 256
    assert p["launches"] == 1 and p["groups_per_split"] == 10 and p["splits"] == 3
    assert w4.explain(1024, 2560, 2048)["stream_k"] == 0
    assert w4.explain(64, 40, 128, path=w4.Path.GEMM_STREAMK)["workgroups"] == 1
    for bad in (dict(bits=2), dict(act=7), dict(path=9)):
        with pytest.raises(ValueError):
            w4.explain(4, 2048, 2048, **bad)
    with pytest.raises(ValueError):
        w4.explain(4, 2048, 100)


@pytest.mark.parametrize("t", __import__("tests.gemm_tilings", fromlist=["STREAMK_TILINGS"]).STREAMK_TILINGS,
                         ids=__import__("tests.gemm_tilings", fromlist=["streamk_id"]).streamk_id)
def test_streamk_shapes_take_their_cut(lib, t):
    """Each stream-K test shape takes its tile, one run per CU, and its kind
    of cut: runs that each lie inside a tile (P slots) or runs that cross
    tile ends (2 P slots), several runs sharing a tile."""
    bits, tm, tn, inside, (m, n, k) = t
    p = w4.explain(m, n, k, path=w4.Path.GEMM_STREAMK, bits=bits)
    assert (p["stream_k"], p["tile_m"], p["tile_n"], p["launches"], p["workgroups"]) == (1, tm, tn, 1, 256), p
    groups = k // 128
    units = -(-m // tm) * -(-n // tn) * groups
    assert (units % 256 == 0 and groups % (units // 256) == 0) == inside
    assert p["splits"] >= (4 if inside else 3), p
    assert p["workspace_bytes"] == (1 << 20) + (1 if inside else 2) * 256 * tm * tn * 4


@pytest.mark.parametrize("t", __import__("tests.gemm_tilings", fromlist=["TILINGS"]).TILINGS,
                         ids=__import__("tests.gemm_tilings", fromlist=["tiling_id"]).tiling_id)
def test_gemm_tiling_shapes_take_their_tiling(lib, t):
    """The GPU tiling tests reach every tiling the planner can pick: each
    listed shape takes exactly its tiling, so a planner change that moves one
    fails here instead of silently dropping coverage."""
    bits, waves, tm, tn, split, (m, n, k) = t
    p = w4.explain(m, n, k, path=w4.Path.GEMM, bits=bits)
    assert (p["waves"], p["tile_m"], p["tile_n"], p["splits"] > 1) == (waves, tm, tn, split), p
