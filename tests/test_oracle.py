"""The CPU oracle against its pins (no GPU).

The oracle is test infrastructure: these tests are what make it trustworthy.
Each pin is described in ``tests/oracle_pins.py``.  The mutation test plants
plausible mistakes into copies of the oracle's C source (on the CPU, in a
child process) and checks that at least one pin fails for every one of them.
"""
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
import synth
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return oracle.oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


@pytest.mark.parametrize("name", ["c1_m1_k1024_n1024", "c2_down_m50_k4096_n1024",
                                  "c3_qkv_m1_k2048_n2560", "c5_m1_k1024_n4096"])
def test_invariants_on_workload_weights(lib, name):
    """The invariants hold on each workload's own weights (outliers, zero groups)."""
    c = synth.case_by_name(name)
    w = synth.make_weight(c).numpy()
    oracle_pins.pin_invariants(lib, w=w)


def test_bf16_and_f16_weights_upcast_exactly(lib):
    """16-bit weights quantize exactly like their FP32 widening."""
    import torch
    rng = np.random.default_rng(2)
    w32 = torch.from_numpy((rng.standard_normal((8, 256)) * 0.02).astype(np.float32))
    for tdt, tag in ((torch.bfloat16, oracle.BF16), (torch.float16, oracle.F16)):
        w16 = w32.to(tdt)
        bits = w16.view(torch.int16).numpy().view(np.uint16)
        q16, s16 = oracle.quantize(bits, tag)
        q32, s32 = oracle.quantize(w16.to(torch.float32).numpy())
        assert np.array_equal(q16, q32) and np.array_equal(s16, s32)


def test_rejects_bad_group_size(lib):
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 200), dtype=np.float32))


# (description, text in w4a16_oracle.c, replacement) -- each is a plausible slip.
MUTANTS = [
    ("divisor 8 instead of 7", "onto code 7 */\n            float scale = amax / 7.0f;",
     "onto code 7 */\n            float scale = amax / 8.0f;"),
    ("divisor 7.5", "onto code 7 */\n            float scale = amax / 7.0f;",
     "onto code 7 */\n            float scale = amax / 7.5f;"),
    ("ties away from zero", "float r = nearbyintf(ratio);", "float r = roundf(ratio);"),
    ("truncation", "float r = nearbyintf(ratio);", "float r = truncf(ratio);"),
    ("reciprocal multiply", "float ratio = weight_as_float(w, w_dtype, row * ldw + kk) / scale;",
     "float ratio = weight_as_float(w, w_dtype, row * ldw + kk) * (1.0f / scale);"),
    ("signed max instead of magnitude", "float a = fabsf(weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j));",
     "float a = weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j);"),
    ("clamp at 6", "if (r > 7.0f)\n                        r = 7.0f;", "if (r > 6.0f)\n                        r = 6.0f;"),
    ("group of 64 for the absmax", "for (int64_t j = 0; j < ORACLE_GROUP; ++j) {\n                float a",
     "for (int64_t j = 0; j < 64; ++j) {\n                float a"),
    ("nibbles swapped", "codes[row * (k / 2) + j] = (uint8_t)(lo | (hi << 4));",
     "codes[row * (k / 2) + j] = (uint8_t)(hi | (lo << 4));"),
    ("no sign extension", "q[row * k + kk] = (int8_t)(v >= 8 ? v - 16 : v);", "q[row * k + kk] = (int8_t)v;"),
    ("scale index by k % 128", "double wv = (double)q[j * k + kk] * (double)s[j * groups + kk / ORACLE_GROUP];",
     "double wv = (double)q[j * k + kk] * (double)s[j * groups + (kk % ORACLE_GROUP) % groups];"),
    ("transposed weight", "double wv = (double)q[j * k + kk] *", "double wv = (double)q[(kk % n_) * k + j] *"),
    ("dropped last term", "for (int64_t kk = 0; kk < k; ++kk) {\n        double xv", "for (int64_t kk = 0; kk < k - 1; ++kk) {\n        double xv"),
    ("bias dropped", "acc += decode16(bias[j], x_dtype);", "acc += 0.0;"),
    ("bias sign", "acc += decode16(bias[j], x_dtype);", "acc -= decode16(bias[j], x_dtype);"),
    ("fp16 exponent bias", "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    ("fp16 subnormal scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("bf16 decoded as fp16", "return dtype == ORACLE_BF16 ? oracle_bf16_to_double(bits) : oracle_f16_to_double(bits);",
     "return oracle_f16_to_double(bits);"),
    ("zero guard missing", "if (scale != 0.0f) {\n                    float ratio", "if (1) {\n                    float ratio"),
    ("dequant drops the scale", "w_hat[row * k + kk] = (double)q[row * k + kk] * (double)s[row * groups + kk / ORACLE_GROUP];",
     "w_hat[row * k + kk] = (double)q[row * k + kk];"),
    ("x row stride ignored", "double xv = decode16(x[i * ldx + kk], x_dtype);", "double xv = decode16(x[kk], x_dtype);"),
    ("swiglu halves swapped", "double up = decode16(x[i * ldx + j], x_dtype);\n                double gate = decode16(x[i * ldx + k + j], x_dtype);",
     "double up = decode16(x[i * ldx + k + j], x_dtype);\n                double gate = decode16(x[i * ldx + j], x_dtype);"),
    ("swiglu row stride taken as 2k", "double up = decode16(x[i * ldx + j], x_dtype);", "double up = decode16(x[i * 2 * k + j], x_dtype);"),
    ("sigmoid sign", "return up * (v / (1.0 + exp(-v)));", "return up * (v / (1.0 + exp(v)));"),
    ("gelu cubic coefficient", "const double u = sqrt(2.0 / M_PI) * (v + 0.044715 * v * v * v);",
     "const double u = sqrt(2.0 / M_PI) * (v + 0.04715 * v * v * v);"),
    ("gelu scale sqrt(1/pi)", "const double u = sqrt(2.0 / M_PI) * (v + 0.044715 * v * v * v);",
     "const double u = sqrt(1.0 / M_PI) * (v + 0.044715 * v * v * v);"),
    ("gelu tanh argument not doubled", "return v / (1.0 + exp(-2.0 * u));", "return v / (1.0 + exp(-u));"),
    ("round16 ties away from zero", "double units = nearbyint(ldexp(a, -q));", "double units = round(ldexp(a, -q));"),
    ("round16 truncates", "double units = nearbyint(ldexp(a, -q));", "double units = trunc(ldexp(a, -q));"),
    ("bf16 with 7 significant bits", "const int p = dtype == ORACLE_BF16 ? 8 : 11;", "const int p = dtype == ORACLE_BF16 ? 7 : 11;"),
    ("fp16 normal range from 2^-15", "const int emin = dtype == ORACLE_BF16 ? -126 : -14;",
     "const int emin = dtype == ORACLE_BF16 ? -126 : -15;"),
    ("no overflow to infinity", "if (r >= ldexp(1.0, emax + 1))\n        return inf;", "if (0)\n        return inf;"),
    ("splitmix64 increment", "uint64_t z = seed + (e + 1) * 0x9E3779B97F4A7C15ull;",
     "uint64_t z = seed + (e + 1) * 0x9E3779B97F4A7C13ull;"),
    ("draw index off by one", "uint64_t z = seed + (e + 1) * 0x9E3779B97F4A7C15ull;",
     "uint64_t z = seed + e * 0x9E3779B97F4A7C15ull;"),
    ("uniform from the low bits", "return (float)(oracle_splitmix64(seed, e) >> 40) * 0x1p-24f;",
     "return (float)(oracle_splitmix64(seed, e) & 0xFFFFFF) * 0x1p-24f;"),
    ("round up when u <= frac", "code = (int)lo + (u < frac ? 1 : 0);", "code = (int)lo + (u <= frac ? 1 : 0);"),
    ("round up with probability 1 - frac", "code = (int)lo + (u < frac ? 1 : 0);", "code = (int)lo + (u < 1.0f - frac ? 1 : 0);"),
    ("truncation instead of floor", "const float lo = floorf(v);", "const float lo = truncf(v);"),
    ("column-major draw offsets", "const float u = oracle_uniform(seed, (uint64_t)(row * k + kk));",
     "const float u = oracle_uniform(seed, (uint64_t)(kk * n + row));"),
    ("alpha on the old weight", "w[j] = fmaf(alpha, p, bd);", "w[j] = fmaf(alpha, bd, p);"),
    ("beta ignored", "const float bd = beta * d;", "const float bd = d;"),
    ("low-rank index transposed", "p = fmaf(update_value(mat1, u_dtype, row * rank + r),",
     "p = fmaf(update_value(mat1, u_dtype, r * n + row),"),
    ("low-rank sum in descending order", "for (int64_t r = 0; r < rank; ++r)\n                        p = fmaf(",
     "for (int64_t r = rank - 1; r >= 0; --r)\n                        p = fmaf("),
    ("dense update row stride ignored", "p = update_value(upd, u_dtype, row * ldu + kk);",
     "p = update_value(upd, u_dtype, row * k + kk);"),
    ("stochastic outside the interior", "if (has_seed && lo >= (float)qmin && lo + 1.0f <= (float)qmax) {",
     "if (has_seed) {"),
    ("stochastic up to the top code", "lo + 1.0f <= (float)qmax) {", "lo <= (float)qmax) {"),
    ("update int8 range taken as int4", "const int qmax = bits == 8 ? 127 : 7;", "const int qmax = 7;"),
    ("update int8 divisor 128", "const int qmax = bits == 8 ? 127 : 7;", "const int qmax = bits == 8 ? 128 : 7;"),
    ("int8 divisor 128", "onto code 127 */\n            float scale8 = amax / 127.0f;",
     "onto code 127 */\n            float scale8 = amax / 128.0f;"),
    ("int8 divisor 255", "onto code 127 */\n            float scale8 = amax / 127.0f;",
     "onto code 127 */\n            float scale8 = amax / 255.0f;"),
    ("int8 ties away from zero", "float r8 = nearbyintf(", "float r8 = roundf("),
    ("int8 truncation", "float r8 = nearbyintf(", "float r8 = truncf("),
    ("int8 clamp at 126", "if (r8 > 127.0f)\n                        r8 = 127.0f;",
     "if (r8 > 126.0f)\n                        r8 = 126.0f;"),
    ("int8 signed max", "float mag = fabsf(weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j));",
     "float mag = weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j);"),
    ("int8 absmax over the first group", "float mag = fabsf(weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j));",
     "float mag = fabsf(weight_as_float(w, w_dtype, row * ldw + j));"),
    ("int8 codes written to the group start", "q[row * k + kk] = (int8_t)code8;", "q[row * k + g * ORACLE_GROUP] = (int8_t)code8;"),
    ("update scale divisor qmax + 1", "const float scale = amax / (float)qmax;",
     "const float scale = amax / (float)(qmax + 1);"),
]

_RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
from oracle import oracle as O
from tests import oracle_pins
lib = O.load({path!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:  # a pin caught the mutant (or the mutant broke)
        failed.append(pin.__name__)
        if {stop_first!r}:
            break
print("FAILED:" + ",".join(failed))
"""


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(desc, old, new):
    src = open(os.path.join(ROOT, "oracle", "w4a16_oracle.c")).read()
    assert src.count(old) == 1, f"mutation site not found exactly once: {desc}"
    mutated = src.replace(old, new)
    if "n_" in new:  # the transposed-index mutant needs the row count in scope
        mutated = mutated.replace("static double one_output(", "static int64_t n_ = 1;\nstatic double one_output(", 1)
        mutated = mutated.replace("#pragma omp parallel for collapse(2) schedule(static)\n    for (int64_t i = 0; i < m; ++i)",
                                  "n_ = n < k ? n : k;\n#pragma omp parallel for collapse(2) schedule(static)\n    for (int64_t i = 0; i < m; ++i)", 1)
    with tempfile.TemporaryDirectory() as d:
        src_path = os.path.join(d, "mutant.c")
        so_path = os.path.join(d, "libmutant.so")
        with open(src_path, "w") as f:
            f.write(mutated)
        oracle.build(src=src_path, out=so_path, extra_flags=["-w"])
        proc = subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT, path=so_path, stop_first=True)],
                              capture_output=True, text=True, timeout=300)
    line = [ln for ln in proc.stdout.splitlines() if ln.startswith("FAILED:")]
    if proc.returncode != 0 and not line:
        return  # the mutant crashed the child: caught
    assert line, proc.stdout + proc.stderr
    caught = [p for p in line[0][len("FAILED:"):].split(",") if p]
    assert caught, f"no pin caught the planted mistake: {desc}"


def test_pins_pass_under_ubsan():
    """The oracle built with the undefined-behaviour sanitizer (aborting on the
    first report) passes every pin: no overflow, shift or conversion UB on
    the paths the pins exercise."""
    with tempfile.TemporaryDirectory() as d:
        so_path = os.path.join(d, "libubsan_oracle.so")
        oracle.build(out=so_path, extra_flags=["-fsanitize=undefined", "-fno-sanitize-recover=all", "-g"])
        proc = subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT, path=so_path, stop_first=False)],
                              capture_output=True, text=True, timeout=600)
    line = [ln for ln in proc.stdout.splitlines() if ln.startswith("FAILED:")]
    assert proc.returncode == 0 and line == ["FAILED:"], proc.stdout[-2000:] + proc.stderr[-2000:]
