"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes a loaded oracle library (``oracle.oracle.load(path)``) and
raises AssertionError on a mismatch.  They are run on the real oracle by
``test_oracle.py`` and on deliberately broken copies of the oracle (mutants,
built on the CPU) to show that each plausible mistake is caught.

What each pin checks against:
  * hand-worked INT4 and INT8 groups and bytes (tests/golden/), worked from
    the method's definition by hand;
  * exact rational arithmetic (tests/exact.py): the correctly rounded FP32
    scale and quotient, and a brute-force nearest-code search;
  * closed forms: identity-like weights give y = c*x exactly, and integer
    weights and activations give an exact integer matrix product;
  * a library routine: numpy's float64 matmul on the dequantized weights;
  * numpy/torch decoders for every 16-bit pattern;
  * the fused activations: torch's float64 silu and tanh-GELU (library
    routines), their odd-part identity, and exact rational rounding of the
    activated value to bf16/fp16 (also against torch/numpy FP32 conversions);
  * weight updates: exactly emulated FP32 steps fed to the (pinned)
    quantizer, identities on dyadic weights, the published SplitMix64
    outputs, and the stochastic rounding's adjacency, offsets,
    reproducibility and unbiasedness.
"""
from __future__ import annotations

import ctypes
import os
from fractions import Fraction

import numpy as np

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class _LazyTorch:
    """torch, imported on first use: the quantizer pins do not need it, and
    the mutation test runs the pins in many short child processes."""

    def __getattr__(self, name):
        import torch as _t
        return getattr(_t, name)


torch = _LazyTorch()


def _read_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _pairs(text, conv):
    out = {}
    for tok in text.split():
        i, v = tok.split(":")
        out[int(i)] = conv(v)
    return out


def pin_hand_worked_groups(lib):
    """Golden: hand-worked RTN groups (ties to even, s = amax/7, zero group)."""
    for line in _read_lines("rtn_hand_worked.txt"):
        name, wtxt, stxt, qtxt = [p.strip() for p in line.split("|")]
        w = np.zeros((1, 128), dtype=np.float32)
        for i, v in _pairs(wtxt, float).items():
            w[0, i] = np.float32(v)
        want_q = np.zeros(128, dtype=np.int8)
        for i, v in _pairs(qtxt, int).items():
            want_q[i] = v
        q, s = oracle.quantize(w, lib=lib)
        assert s[0, 0] == np.float32(stxt), f"{name}: scale {s[0,0]!r} != {stxt}"
        assert np.array_equal(q[0], want_q), f"{name}: codes {q[0][:16]} != {want_q[:16]}"
        if float(stxt) == 0.0:
            assert np.signbit(s[0, 0]) == False, f"{name}: zero scale must be +0"  # noqa: E712


def pin_negative_zero_group(lib):
    """A group of -0.0 values quantizes like an all-zero group: s = +0, q = 0."""
    w = np.full((2, 256), -0.0, dtype=np.float32)
    w[1, 128:] = 0.0
    q, s = oracle.quantize(w, lib=lib)
    assert np.all(q == 0)
    assert np.all(s == 0) and not np.any(np.signbit(s)), s


def pin_canonical_nibbles(lib):
    """Golden: hand-worked canonical byte layout, and its inverse."""
    for line in _read_lines("canonical_nibbles.txt"):
        ctxt, btxt = [p.strip() for p in line.split("|")]
        q = np.array([int(v) for v in ctxt.split()], dtype=np.int8)[None, :]
        want = np.array([int(v, 16) for v in btxt.split()], dtype=np.uint8)[None, :]
        got = oracle.codes_to_nibbles(q, lib=lib)
        assert np.array_equal(got, want), f"{got} != {want}"
        back = oracle.nibbles_to_codes(want, lib=lib)
        assert np.array_equal(back, q), f"{back} != {q}"


def _check_exact_rtn(w, q, s, qmax, lo, hi):
    """Returns the number of codes that differ from the brute-force nearest code
    (each only where the quotient is within one FP32 ulp of a half-integer)."""
    n, k = w.shape
    near_ties = 0
    for r in range(n):
        for g in range(k // 128):
            seg = w[r, g * 128:(g + 1) * 128]
            amax = max(abs(exact.f32_fraction(v)) for v in seg)
            want_s = exact.round_to_f32(amax / qmax)
            assert float(s[r, g]) == want_s, (r, g, float(s[r, g]), want_s)
            sf = Fraction(want_s)
            for j, v in enumerate(seg):
                wf = exact.f32_fraction(v)
                got = int(q[r, g * 128 + j])
                if sf == 0:
                    assert got == 0
                    continue
                ratio = wf / sf
                quotient = exact.round_to_f32(ratio)
                want = max(lo, min(hi, exact.round_half_even(Fraction(quotient))))
                assert got == want, (r, g, j, got, want)
                # |w - c s| is convex in c, so the nearest code lies within two
                # of the clamped rounded ratio: search that window exhaustively
                c = max(lo, min(hi, int(ratio)))
                brute = exact.argmin_code(wf, sf, max(lo, c - 2), min(hi, c + 2))
                if brute != got:
                    half = Fraction(2 * exact.round_half_even(ratio - Fraction(1, 2)) + 1, 2)
                    assert abs(ratio - half) <= exact.ulp_f32(float(ratio)), (r, g, j, got, brute)
                    near_ties += 1
    return near_ties


def _planted_weights(seed, n, k, top):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    # a group with planted exact and near half-integer quotients
    w[0, :128] = 0.0
    w[0, 0] = np.float32(0.7)
    w[0, 1:8] = np.float32(0.7) * np.arange(1, 8, dtype=np.float32) / np.float32(2 * top)
    w[1, 128:256] *= np.float32(1e-38)  # subnormal magnitudes
    return w


def pin_exact_scales_and_codes(lib, seed=11, n=24, k=384):
    """Exact rationals: s is amax/7 correctly rounded to FP32; each code is the
    ties-to-even rounding of the correctly rounded FP32 quotient; brute-force
    nearest codes differ only where the quotient lies within one FP32 ulp of a
    half-integer."""
    w = _planted_weights(seed, n, k, 7)
    q, s = oracle.quantize(w, lib=lib)
    assert _check_exact_rtn(w, q, s, 7, -8, 7) <= 3


def pin_invariants(lib, w=None, seed=5):
    """Codes in [-7, 7]; |w - q s| <= s (1/2 + 2^-21); every nonzero group has a
    code of magnitude 7; zero groups give s = +0 and q = 0; quantize(-w) = (-q, s);
    quantize(2^j w) = (q, 2^j s)."""
    if w is None:
        rng = np.random.default_rng(seed)
        w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
        w[3, 256:384] = 0.0
        w[7, :] = 0.0
        mask = rng.random(w.shape) < 0.01
        w[mask] = (rng.standard_normal(mask.sum()) * 0.2).astype(np.float32)
    n, k = w.shape
    q, s = oracle.quantize(w, lib=lib)
    assert q.min() >= -7 and q.max() <= 7, (q.min(), q.max())
    s_full = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s_full)
    assert np.all(err <= s_full * (0.5 + 2.0 ** -21)), float((err / np.maximum(s_full, 1e-300)).max())
    qg = np.abs(q.reshape(n, k // 128, 128)).max(axis=2)
    zero = np.all(w.reshape(n, k // 128, 128) == 0, axis=2)
    assert np.all(qg[~zero] == 7)
    assert np.all(s[zero] == 0) and not np.any(np.signbit(s[zero]))
    assert np.all(q.reshape(n, k // 128, 128)[zero] == 0)
    qn, sn = oracle.quantize(-w, lib=lib)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for j in (5, -5):
        f = np.float32(2.0 ** j)
        qj, sj = oracle.quantize(w * f, lib=lib)
        assert np.array_equal(qj, q) and np.array_equal(sj, s * f)


def pin_int8_hand_worked_groups(lib):
    """Golden: hand-worked RTN INT8 groups (ties to even, s = amax/127, zero group)."""
    for line in _read_lines("rtn8_hand_worked.txt"):
        name, wtxt, stxt, qtxt = [p.strip() for p in line.split("|")]
        w = np.zeros((1, 128), dtype=np.float32)
        for i, v in _pairs(wtxt, float).items():
            w[0, i] = np.float32(v)
        want_q = np.zeros(128, dtype=np.int8)
        for i, v in _pairs(qtxt, int).items():
            want_q[i] = v
        q, s = oracle.quantize_int8(w, lib=lib)
        assert s[0, 0] == np.float32(stxt), f"{name}: scale {s[0,0]!r} != {stxt}"
        assert np.array_equal(q[0], want_q), f"{name}: codes {q[0][:16]} != {want_q[:16]}"


def pin_int8_exact_scales_and_codes(lib, seed=12, n=16, k=384):
    """Exact rationals for INT8: s is amax/127 correctly rounded to FP32; each
    code is the ties-to-even rounding of the correctly rounded FP32 quotient,
    and equals the brute-force nearest code in [-128, 127] except within one
    FP32 ulp of a half-integer."""
    w = _planted_weights(seed, n, k, 127)
    q, s = oracle.quantize_int8(w, lib=lib)
    assert _check_exact_rtn(w, q, s, 127, -128, 127) <= 3


def pin_int8_invariants(lib, w=None, seed=6):
    """INT8 codes in [-127, 127]; |w - q s| <= s (1/2 + 2^-16); every nonzero
    group has a code of magnitude 127; zero groups give s = +0 and q = 0;
    quantize(-w) = (-q, s); quantize(2^j w) = (q, 2^j s); the INT8 scale is the
    INT4 scale times 7/127 up to FP32 rounding."""
    if w is None:
        rng = np.random.default_rng(seed)
        w = (rng.standard_normal((48, 1024)) * 0.02).astype(np.float32)
        w[3, 256:384] = 0.0
        w[5, :] = -0.0
        mask = rng.random(w.shape) < 0.01
        w[mask] = (rng.standard_normal(mask.sum()) * 0.2).astype(np.float32)
    n, k = w.shape
    q, s = oracle.quantize_int8(w, lib=lib)
    assert q.min() >= -127 and q.max() <= 127, (q.min(), q.max())
    s_full = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s_full)
    assert np.all(err <= s_full * (0.5 + 2.0 ** -16)), float((err / np.maximum(s_full, 1e-300)).max())
    qg = np.abs(q.reshape(n, k // 128, 128).astype(np.int32)).max(axis=2)
    zero = np.all(w.reshape(n, k // 128, 128) == 0, axis=2)
    assert np.all(qg[~zero] == 127)
    assert np.all(s[zero] == 0) and not np.any(np.signbit(s[zero]))
    assert np.all(q.reshape(n, k // 128, 128)[zero] == 0)
    qn, sn = oracle.quantize_int8(-w, lib=lib)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for j in (5, -5):
        f = np.float32(2.0 ** j)
        qj, sj = oracle.quantize_int8(w * f, lib=lib)
        assert np.array_equal(qj, q) and np.array_equal(sj, s * f)
    _, s4 = oracle.quantize(w, lib=lib)
    ratio = s.astype(np.float64)[~zero] * 127 / (s4.astype(np.float64)[~zero] * 7)
    assert np.all(np.abs(ratio - 1) < 2.0 ** -22), float(np.abs(ratio - 1).max())


def pin_decoders(lib):
    """bf16 and fp16 decoding agrees with torch/numpy for all 65536 patterns."""
    bits = np.arange(65536, dtype=np.uint16)
    want_f16 = bits.view(np.float16).astype(np.float64)
    want_bf16 = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    # sample every pattern through the C entry points (cheap: scalar calls)
    got_f16 = np.array([lib.oracle_f16_to_double(int(b)) for b in bits])
    got_bf16 = np.array([lib.oracle_bf16_to_double(int(b)) for b in bits])
    for got, want in ((got_f16, want_f16), (got_bf16, want_bf16)):
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_identity_like(lib):
    """W = c I with c = 7 * 2^-3: s = 2^-3 on the diagonal groups, q = 7 on the
    diagonal, every other group all-zero, so y = c x exactly (bf16 and fp16)."""
    n = 384
    c = np.float32(7.0 * 2.0 ** -3)
    w = np.zeros((n, n), dtype=np.float32)
    np.fill_diagonal(w, c)
    q, s = oracle.quantize(w, lib=lib)
    rng = np.random.default_rng(3)
    for tag, tdt in ((oracle.BF16, torch.bfloat16), (oracle.F16, torch.float16)):
        x = torch.from_numpy(rng.standard_normal((5, n)).astype(np.float32)).to(tdt)
        xb = x.view(torch.int16).numpy().view(np.uint16)
        y = oracle.linear(xb, tag, q, s, lib=lib)
        want = x.to(torch.float64).numpy() * float(c)
        assert np.array_equal(y, want), float(np.abs(y - want).max())


def pin_exact_integer_gemm(lib, seed=9):
    """W = q_int 2^-3 with one |q| = 7 per group, x and bias small integers: the
    layer output is an exact integer matrix product (numpy int64) times 2^-3."""
    rng = np.random.default_rng(seed)
    m, k, n = 6, 512, 40
    qi = rng.integers(-7, 8, size=(n, k))
    qi[:, ::128] = 7 * np.where(rng.random((n, k // 128)) < 0.5, 1, -1)
    w = (qi * 2.0 ** -3).astype(np.float32)
    q, s = oracle.quantize(w, lib=lib)
    assert np.array_equal(q, qi.astype(np.int8))
    assert np.all(s == np.float32(2.0 ** -3))
    xi = rng.integers(-4, 5, size=(m, k))
    bi = rng.integers(-9, 10, size=n)
    for tag, tdt in ((oracle.BF16, torch.bfloat16), (oracle.F16, torch.float16)):
        xb = torch.from_numpy(xi.astype(np.float32)).to(tdt).view(torch.int16).numpy().view(np.uint16)
        bb = torch.from_numpy(bi.astype(np.float32)).to(tdt).view(torch.int16).numpy().view(np.uint16)
        y = oracle.linear(xb, tag, q, s, bb, lib=lib)
        want = (xi @ qi.T) * 2.0 ** -3 + bi
        assert np.array_equal(y, want.astype(np.float64)), float(np.abs(y - want).max())
        ent = oracle.linear_entries(xb, tag, q, s, bb, np.array([0, 5, 3]), np.array([39, 0, 17]), lib=lib)
        assert np.array_equal(ent, want[[0, 5, 3], [39, 0, 17]].astype(np.float64))


def pin_matches_library_matmul(lib, seed=4):
    """Random case: the oracle equals numpy's float64 matmul of the dequantized
    weight (plus bias) to float64 rounding."""
    rng = np.random.default_rng(seed)
    m, k, n = 7, 640, 96
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = oracle.quantize(w, lib=lib)
    w_hat = oracle.dequantize(q, s, lib=lib)
    want_hat = q.astype(np.float64) * np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.array_equal(w_hat, want_hat)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((rng.standard_normal(n) * 0.01).astype(np.float32)).to(torch.bfloat16)
    y = oracle.linear(x.view(torch.int16).numpy().view(np.uint16), oracle.BF16, q, s,
                      b.view(torch.int16).numpy().view(np.uint16), lib=lib)
    xd = x.to(torch.float64).numpy()
    want = xd @ want_hat.T + b.to(torch.float64).numpy()
    bound = 1e-13 * (np.abs(xd) @ np.abs(want_hat).T + 1.0)
    assert np.all(np.abs(y - want) <= bound)


def _decode(bits: int, tag: int) -> float:
    arr = np.array([bits], dtype=np.uint16)
    if tag == oracle.F16:
        return float(arr.view(np.float16)[0])
    return float(torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)[0])


def pin_round16_exact(lib, seed=21):
    """Rounding a double to bf16/fp16 equals the exact rational nearest-even
    rounding (tests/exact.py), over random magnitudes from the subnormal range
    to overflow, exact ties, and the edges of both formats."""
    rng = np.random.default_rng(seed)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-150, 130, 400)))
    vals += [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25,
             3 * 2.0 ** -26, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8,
             1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 3.3895313892515355e38, 3.4e38, -1e-30]
    for tag, fmt in ((oracle.BF16, "bf16"), (oracle.F16, "f16")):
        for v in vals:
            got = _decode(lib.oracle_round16(float(v), tag), tag)
            want = exact.round_to_16(Fraction(float(v)), fmt)
            assert got == want and np.signbit(got) == np.signbit(v), (fmt, v, got, want)


def pin_round16_matches_fp32_conversion(lib, seed=22):
    """For every binary32 value (random bit patterns) the rounding equals the
    libraries' own single-rounding conversions: torch float32 -> bfloat16 and
    numpy float32 -> float16."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want_bf = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    with np.errstate(over="ignore"):
        want_h = f.astype(np.float16).view(np.uint16)
    for i, v in enumerate(f):
        assert lib.oracle_round16(float(v), oracle.BF16) == want_bf[i], (float(v), hex(want_bf[i]))
        assert lib.oracle_round16(float(v), oracle.F16) == want_h[i], (float(v), hex(want_h[i]))


def pin_activation_library(lib):
    """The activations agree with torch's float64 silu and tanh-approximate GELU
    on a grid from -40 to 40 (library routines), to 1e-14 relative plus
    1e-15 |x| absolute (torch evaluates 1 + tanh(u), which cancels for large
    negative x)."""
    grid = np.concatenate([np.linspace(-40, 40, 801), [0.0, 1e-8, -1e-8, 0.5, -3.25, 6.0]])
    t = torch.from_numpy(grid)
    silu = torch.nn.functional.silu(t).numpy()
    gelu = torch.nn.functional.gelu(t, approximate="tanh").numpy()
    for i, v in enumerate(grid):
        for up in (1.0, -2.5):
            got = lib.oracle_act_value(float(v), up, oracle.ACT_SWIGLU)
            assert abs(got - up * silu[i]) <= 1e-14 * abs(up * silu[i]) + 1e-15 * abs(up * v), (v, up, got)
        got = lib.oracle_act_value(float(v), 0.0, oracle.ACT_GELU_TANH)
        assert abs(got - gelu[i]) <= 1e-14 * abs(gelu[i]) + 1e-15 * abs(v), (v, got, gelu[i])


def pin_activation_odd_part(lib):
    """Both activations have odd part x/2 (their gates are logistic-type): silu(x) -
    silu(-x) = x and gelu(x) - gelu(-x) = x; silu(0) = gelu(0) = 0."""
    for v in (0.25, 1.0, 2.75, 7.5, 19.0):
        s = lib.oracle_act_value(v, 1.0, oracle.ACT_SWIGLU) - lib.oracle_act_value(-v, 1.0, oracle.ACT_SWIGLU)
        g = lib.oracle_act_value(v, 0.0, oracle.ACT_GELU_TANH) - lib.oracle_act_value(-v, 0.0, oracle.ACT_GELU_TANH)
        assert abs(s - v) <= 4e-16 * v and abs(g - v) <= 4e-16 * v, (v, s, g)
    assert lib.oracle_act_value(0.0, 3.0, oracle.ACT_SWIGLU) == 0.0
    assert lib.oracle_act_value(0.0, 0.0, oracle.ACT_GELU_TANH) == 0.0


def pin_activate_rows(lib, seed=23):
    """The activated input takes up from the first half of a SwiGLU row and
    gate from the second, reads GELU rows in place, honours the row stride,
    and rounds each value once: equal to torch's float64 activation followed
    by the exact rounding, element by element."""
    rng = np.random.default_rng(seed)
    m, k = 3, 256
    for tag, tdt, fmt in ((oracle.BF16, torch.bfloat16, "bf16"), (oracle.F16, torch.float16, "f16")):
        x = torch.from_numpy((rng.standard_normal((m, 2 * k + 8)) * 3).astype(np.float32)).to(tdt)
        x[0, :4] = torch.tensor([3.0, -2.0, 0.5, 0.0], dtype=tdt)          # up values
        x[0, k:k + 4] = torch.tensor([30.0, 0.0, -30.0, 5.0], dtype=tdt)   # gate values
        xb = x.view(torch.int16).numpy().view(np.uint16)
        xd = x.to(torch.float64)
        up, gate = xd[:, :k], xd[:, k:2 * k]
        want_sw = (up * torch.nn.functional.silu(gate)).numpy()
        got = oracle.activate(xb[:, :2 * k], tag, oracle.ACT_SWIGLU, lib=lib)
        for i in range(m):
            for j in range(k):
                assert _decode(got[i, j], tag) == exact.round_to_16(Fraction(float(want_sw[i, j])), fmt), (i, j)
        # silu(30) = 30 (1 - 9e-14): up 3 with gate 30 gives 90 after rounding
        # (swapped halves would give 30 silu(3) = 85.7); gate 0 gives an exact zero
        assert _decode(got[0, 0], tag) == 90.0 and _decode(got[0, 1], tag) == 0.0
        # GELU inputs within [-3, 3], where torch's 1 + tanh(u) is accurate
        xg = x[:, :k].clamp(-3.0, 3.0)
        want_ge = torch.nn.functional.gelu(xg.to(torch.float64), approximate="tanh").numpy()
        got = oracle.activate(xg.view(torch.int16).numpy().view(np.uint16), tag, oracle.ACT_GELU_TANH, lib=lib)
        for i in range(m):
            for j in range(k):
                assert _decode(got[i, j], tag) == exact.round_to_16(Fraction(float(want_ge[i, j])), fmt), (i, j)
        # a row stride wider than the row: the C entry point with ldx = 2k + 8
        out = np.empty((m, k), dtype=np.uint16)
        xs = np.ascontiguousarray(xb)
        rc = lib.oracle_activate(xs.ctypes.data_as(ctypes.c_void_p), tag, oracle.ACT_SWIGLU, m, k, 2 * k + 8,
                                 out.ctypes.data_as(ctypes.c_void_p))
        assert rc == 0
        assert np.array_equal(out, oracle.activate(xb[:, :2 * k], tag, oracle.ACT_SWIGLU, lib=lib))


def pin_splitmix64_published(lib):
    """Golden: the generator's published outputs (tests/golden/splitmix64.txt);
    output i + 1 of a seed is draw i, and a draw's top 24 bits are the uniform."""
    for line in _read_lines("splitmix64.txt"):
        seed, outs = [p.strip() for p in line.split("|")]
        for i, want in enumerate(int(v) for v in outs.split()):
            got = lib.oracle_splitmix64(int(seed), i)
            assert got == want, (seed, i, got, want)
            assert lib.oracle_uniform(int(seed), i) == (want >> 40) * 2.0 ** -24


def _fl32(fr: Fraction) -> Fraction:
    return Fraction(exact.round_to_f32(fr))


def _exact_update(q, s, upd=None, m1=None, m2=None, alpha=1.0, beta=1.0):
    """The update's FP32 steps emulated exactly: each product, sum and fused
    multiply-add computed in rationals and rounded once to binary32."""
    n, k = q.shape
    a, b = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    out = np.empty((n, k), dtype=np.float32)
    for i in range(n):
        for j in range(k):
            d = _fl32(Fraction(int(q[i, j])) * Fraction(float(s[i, j // 128])))
            if upd is not None:
                p = Fraction(float(upd[i, j]))
            else:
                p = Fraction(0)
                for r in range(m1.shape[1]):
                    p = _fl32(Fraction(float(m1[i, r])) * Fraction(float(m2[r, j])) + p)
            out[i, j] = np.float32(exact.round_to_f32(a * p + _fl32(b * d)))
    return out


def _quantizer(bits):
    return oracle.quantize_int8 if bits == 8 else oracle.quantize


def pin_update_matches_exact_steps(lib, seed=31, bits=4):
    """Round-to-nearest updates (dense and low-rank, several alpha/beta) equal
    the quantizer applied to the exactly emulated FP32 steps."""
    rng = np.random.default_rng(seed)
    n, k = 4, 256
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    quant = _quantizer(bits)
    q, s = quant(w, lib=lib)
    upd = (rng.standard_normal((n, k)) * 0.01).astype(np.float32)
    m1 = (rng.standard_normal((n, 3)) * 0.1).astype(np.float32)
    m2 = (rng.standard_normal((3, k)) * 0.1).astype(np.float32)
    for kind in ("dense", "lowrank"):
        for alpha, beta in ((1.0, 1.0), (0.375, 1.0), (-2.0, 0.5)):
            if kind == "dense":
                got = oracle.update(q, s, upd=upd, alpha=alpha, beta=beta, lib=lib, bits=bits)
                wn = _exact_update(q, s, upd=upd, alpha=alpha, beta=beta)
            else:
                got = oracle.update(q, s, mat1=m1, mat2=m2, alpha=alpha, beta=beta, lib=lib, bits=bits)
                wn = _exact_update(q, s, m1=m1, m2=m2, alpha=alpha, beta=beta)
            want = quant(wn, lib=lib)
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), (kind, alpha, beta)
    if bits == 8:
        return
    # a dense update with a row stride wider than the row (the C entry point)
    wide = np.zeros((n, k + 8), dtype=np.float32)
    wide[:, :k] = upd
    wide[:, k:] = 1e3  # never read
    q2, s2 = q.copy(), s.copy()
    rc = lib.oracle_update(q2.ctypes.data_as(ctypes.c_void_p), s2.ctypes.data_as(ctypes.c_void_p), n, k,
                           wide.ctypes.data_as(ctypes.c_void_p), k + 8, None, None, 0, oracle.F32,
                           ctypes.c_float(1.0), ctypes.c_float(1.0), 0, 0, 4)
    assert rc == 0
    want = oracle.update(q, s, upd=upd, lib=lib)
    assert np.array_equal(q2, want[0]) and np.array_equal(s2, want[1])
    # the low-rank sum runs r ascending: terms 1, 2^-24, 2^-24 sum to 1 in that
    # order (each tie rounds to even) but to 1 + 2^-23 in the other; that value
    # is the group's largest, so it shows in the scale
    m1 = np.array([[1.0, 2.0 ** -24, 2.0 ** -24]], dtype=np.float32)
    m2 = np.zeros((3, 128), dtype=np.float32)
    m2[:, 0] = 1.0
    zq, zs = np.zeros((1, 128), np.int8), np.zeros((1, 1), np.float32)
    got = oracle.update(zq, zs, mat1=m1, mat2=m2, lib=lib)
    wn = _exact_update(zq, zs, m1=m1, m2=m2)
    assert wn[0, 0] == 1.0 and got[1][0, 0] == np.float32(1.0) / np.float32(7.0), (wn[0, 0], got[1][0, 0])


def pin_update_identities(lib, seed=32):
    """Dyadic weights (codes times 2^-3): a zero update keeps codes and scales
    in both rounding modes (exact hits are never perturbed); subtracting the
    dequantized weight gives all-zero groups (s = +0, q = 0); doubling it
    doubles the scales and keeps the codes."""
    rng = np.random.default_rng(seed)
    n, k = 6, 384
    qi = rng.integers(-7, 8, size=(n, k))
    qi[:, ::128] = 7
    w = (qi * 2.0 ** -3).astype(np.float32)
    q, s = oracle.quantize(w, lib=lib)
    zero = np.zeros((n, k), dtype=np.float32)
    for sd in (None, 7):
        q2, s2 = oracle.update(q, s, upd=zero, seed=sd, lib=lib)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)
        q3, s3 = oracle.update(q, s, upd=-w, seed=sd, lib=lib)
        assert np.all(q3 == 0) and np.all(s3 == 0) and not np.any(np.signbit(s3))
        q4, s4 = oracle.update(q, s, upd=w, seed=sd, lib=lib)
        assert np.array_equal(q4, q) and np.array_equal(s4, 2 * s)


def pin_update_int8_matches_exact_steps(lib):
    """The INT8 update: the pinned INT8 quantizer on the exactly emulated FP32
    steps (dense and low-rank, several alpha/beta)."""
    pin_update_matches_exact_steps(lib, seed=41, bits=8)


def pin_stochastic_rounding_int8(lib):
    """Stochastic INT8 codes: adjacency, draw offsets, reproducibility,
    unbiasedness and the crafted cases, with the INT8 code range."""
    pin_stochastic_rounding(lib, seed=43, bits=8)


def pin_stochastic_rounding(lib, seed=33, bits=4):
    """Stochastic codes: each is floor(v) or floor(v) + 1 of the exactly
    emulated quotient v (codes outside the interior keep the nearest code),
    element (i, j) rounds up exactly when draw i*K + j of the seed falls below
    v - floor(v), a seed reproduces its result, and over many seeds the mean
    code approaches v (unbiased)."""
    rng = np.random.default_rng(seed)
    n, k = 3, 256
    quant = _quantizer(bits)
    qmax = 127 if bits == 8 else 7
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = quant(w, lib=lib)
    upd = (rng.standard_normal((n, k)) * (0.005 if bits == 4 else 0.0005)).astype(np.float32)
    wn = _exact_update(q, s, upd=upd)
    qn, sn = quant(wn, lib=lib)
    v = np.empty((n, k))
    for i in range(n):
        for j in range(k):
            v[i, j] = exact.round_to_f32(Fraction(float(wn[i, j])) / Fraction(float(sn[i, j // 128])))
    lo = np.floor(v)
    interior = (lo >= -qmax - 1) & (lo + 1 <= qmax)
    trials = []
    for sd in range(300):
        q2, s2 = oracle.update(q, s, upd=upd, seed=sd, lib=lib, bits=bits)
        assert np.array_equal(s2, sn)  # the deterministic scales
        assert np.all(((q2 == lo) | (q2 == lo + 1))[interior])
        assert np.array_equal(q2[~interior], qn[~interior])
        trials.append(q2.astype(np.float64))
    q_a, _ = oracle.update(q, s, upd=upd, seed=12345, lib=lib, bits=bits)
    q_b, _ = oracle.update(q, s, upd=upd, seed=12345, lib=lib, bits=bits)
    assert np.array_equal(q_a, q_b)
    for i in range(n):
        for j in range(k):
            if interior[i, j]:
                up = lib.oracle_uniform(12345, i * k + j) < v[i, j] - lo[i, j]
                assert q_a[i, j] == lo[i, j] + up, (i, j)
    # a quotient equal to its own draw does not round up (u < frac is strict):
    # from an all-zero weight, the dense update itself is w'; qmax fixes s' = 1
    u0 = lib.oracle_uniform(77, 0)
    z = np.zeros((1, 128), dtype=np.float32)
    craft = np.zeros((1, 128), dtype=np.float32)
    craft[0, 0], craft[0, 1] = u0, float(qmax)
    qc, sc = oracle.update(z.astype(np.int8), np.zeros((1, 1), np.float32), upd=craft, seed=77, lib=lib, bits=bits)
    assert sc[0, 0] == 1.0 and qc[0, 0] == 0 and qc[0, 1] == qmax, (qc[0, :2], sc)
    # outside the interior the nearest code stands: a = 1.0000007 gives
    # s' = fl32(a/7) = 0.14285724 and v = 7.0000005 (floor 7, no code 8);
    # for INT8, a = 2.7708886 gives s' = fl32(a/127) and v = 127.00001
    # (floor 127, no code 128); seed 1127518 draws 2 * 2^-24 first, below
    # v - qmax, so a rounding that ignored the code range would step past it
    craft = np.zeros((1, 128), dtype=np.float32)
    craft[0, 0] = np.float32(2.7708886 if bits == 8 else 1.0000007)
    qc, sc = oracle.update(z.astype(np.int8), np.zeros((1, 1), np.float32), upd=craft, seed=1127518, lib=lib,
                           bits=bits)
    assert lib.oracle_uniform(1127518, 0) == 2 * 2.0 ** -24
    assert np.float32(craft[0, 0]) / sc[0, 0] > np.float32(qmax) and qc[0, 0] == qmax, (qc[0, 0], sc[0, 0])
    mean = np.mean(trials, axis=0)
    frac = v - lo
    sd_err = np.sqrt(frac * (1 - frac) / len(trials)) + 1e-6
    assert np.all(np.abs(mean - v)[interior] <= 5 * sd_err[interior] + 1e-6)
    assert np.mean(np.abs(mean - v)[interior]) < 0.02


ALL_PINS = [
    pin_hand_worked_groups,
    pin_negative_zero_group,
    pin_canonical_nibbles,
    pin_exact_scales_and_codes,
    pin_invariants,
    pin_int8_hand_worked_groups,
    pin_int8_exact_scales_and_codes,
    pin_int8_invariants,
    pin_decoders,
    pin_identity_like,
    pin_exact_integer_gemm,
    pin_matches_library_matmul,
    pin_round16_exact,
    pin_round16_matches_fp32_conversion,
    pin_activation_library,
    pin_activation_odd_part,
    pin_activate_rows,
    pin_splitmix64_published,
    pin_update_matches_exact_steps,
    pin_update_identities,
    pin_stochastic_rounding,
    pin_update_int8_matches_exact_steps,
    pin_stochastic_rounding_int8,
]
