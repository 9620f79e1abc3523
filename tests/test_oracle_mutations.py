"""The oracle's pins must catch plausible mistakes.  Each case below compiles a
copy of oracle.c with one planted mistake (on the CPU, in a temporary
directory) and checks that at least one pin in test_oracle.py,
test_oracle_i8.py, test_oracle_epilogue.py or test_oracle_norm.py fails on it."""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle as pins
import test_oracle_epilogue as pins_ep
import test_oracle_i8 as pins_i8
import test_oracle_norm as pins_norm

SRC = oracle.oracle.SRC_PATH

# (name, text in oracle.c, replacement)
MUTATIONS = [
    ("dense-sign", "orc_bf16_value(X[m * K + k]);\n                acc += p;\n                mag += fabs(p);\n            }\n            Y[m * N + n] = acc;\n            if (B) B[m * N + n] = mag;\n        }\n    }\n}\n\n/* Same",
     "orc_bf16_value(X[m * K + k]);\n                acc -= p;\n                mag += fabs(p);\n            }\n            Y[m * N + n] = acc;\n            if (B) B[m * N + n] = mag;\n        }\n    }\n}\n\n/* Same"),
    ("dense-transposed-W", "orc_bf16_value(W[n * K + k]) * orc_bf16_value(X[m * K + k])",
     "orc_bf16_value(W[k * N + n]) * orc_bf16_value(X[m * K + k])"),
    ("dense-dropped-last-term", "double p = orc_bf16_value(W[n * K + k])",
     "if (k == K - 1) break;\n                double p = orc_bf16_value(W[n * K + k])"),
    ("dense-bound-not-abs", "orc_bf16_value(X[m * K + k]);\n                acc += p;\n                mag += fabs(p);\n            }\n            Y[m * N + n] = acc;\n            if (B) B[m * N + n] = mag;\n        }\n    }\n}\n\n/* Same",
     "orc_bf16_value(X[m * K + k]);\n                acc += p;\n                mag += p;\n            }\n            Y[m * N + n] = acc;\n            if (B) B[m * N + n] = mag;\n        }\n    }\n}\n\n/* Same"),
    ("bf16-exponent-bias", "e - 127 - 7", "e - 127 - 8"),
    ("bf16-subnormal-dropped", "mag = ldexp((double)f, -126 - 7);", "mag = 0.0;"),
    ("f16-subnormal-scale", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("f16-encode-ties-up", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    ("f16-encode-overflow", "if (a >= 65520.0)", "if (a >= 65504.0)"),
    ("q4-nibble-order", "int nib = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "int nib = (k % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    ("q4-sign-encoding", "return (nib ^ 8) - 8;", "return nib - 8;"),
    ("q4-unsigned-codes", "return (nib ^ 8) - 8;", "return nib;"),
    ("q4-group-index", "orc_f16_value(S[n * (K / 64) + k / 64]);\n                double p",
     "orc_f16_value(S[n * (K / 64) + k / 128]);\n                double p"),
    ("q4-dequant-group-index", "orc_f16_value(S[n * (K / 64) + k / 64]);\n}",
     "orc_f16_value(S[n * (K / 64) + (k % 64)]);\n}"),
    ("quant-scale-divisor", "orc_f16_from_f64(a / 7.0)", "orc_f16_from_f64(a / 8.0)"),
    ("quant-clamp-low", "if (r < -8.0) r = -8.0;", "if (r < -7.0) r = -7.0;"),
    ("quant-no-saturation", "if ((sbits & 0x7FFF) == 0x7C00) sbits = 0x7BFF;", ""),
    ("quant-truncating-round", "r = (v < 0.0) ? -round_half_even(-v) : round_half_even(v);\n                        if (r < -8.0)",
     "r = trunc(v);\n                        if (r < -8.0)"),
    ("quant-pack-order", "(uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4))",
     "(uint8_t)((q[1] & 0xF) | ((q[0] & 0xF) << 4))"),
    ("quant-absmax-signed", "double w = fabs(orc_bf16_value(W[n * K + k]));\n                if (w > a) a = w;\n            }\n            uint16_t",
     "double w = orc_bf16_value(W[n * K + k]);\n                if (w > a) a = w;\n            }\n            uint16_t"),
    ("i8-scale-divisor", "(float)(a / 127.0)", "(float)(a / 128.0)"),
    ("i8-truncating-round", "r = (v < 0.0) ? -round_half_even(-v) : round_half_even(v);\n                if (r < -127.0)",
     "r = trunc(v);\n                if (r < -127.0)"),
    ("i8-round-half-up", "r = (v < 0.0) ? -round_half_even(-v) : round_half_even(v);\n                if (r < -127.0)",
     "r = floor(v + 0.5);\n                if (r < -127.0)"),
    ("i8-absmax-signed", "double w = fabs(orc_bf16_value(W[n * K + k]));\n            if (w > a) a = w;\n        }\n        float s",
     "double w = orc_bf16_value(W[n * K + k]);\n            if (w > a) a = w;\n        }\n        float s"),
    ("i8-scale-not-applied", "Y[m * N + n] = (double)S[n] * acc;", "Y[m * N + n] = acc;"),
    ("i8-unsigned-codes", "double p = (double)Wq[n * K + k] * orc_bf16_value",
     "double p = (double)(uint8_t)Wq[n * K + k] * orc_bf16_value"),
    ("silu-sign", "H[i] = G[i] / (1.0 + exp(-G[i])) * U[i];", "H[i] = G[i] / (1.0 + exp(G[i])) * U[i];"),
    ("silu-missing-gate", "H[i] = G[i] / (1.0 + exp(-G[i])) * U[i];", "H[i] = 1.0 / (1.0 + exp(-G[i])) * U[i];"),
    ("residual-dropped", "Y[i] = P[i] + (double)R[i];", "Y[i] = P[i];"),
    ("i8-dequant-scale-index", "Wd[n * K + k] = (double)Wq[n * K + k] * (double)S[n];",
     "Wd[n * K + k] = (double)Wq[n * K + k] * (double)S[k % N];"),
    ("rms-sum-not-mean", "sqrt(ss / (double)K + eps)", "sqrt(ss + eps)"),
    ("rms-eps-dropped", "sqrt(ss / (double)K + eps)", "sqrt(ss / (double)K)"),
    ("rms-no-sqrt", "1.0 / sqrt(ss / (double)K + eps)", "1.0 / (ss / (double)K + eps)"),
    ("rms-gain-dropped", "orc_bf16_value(X[m * K + k]) *\n                                             orc_bf16_value(G[k]) * inv",
     "orc_bf16_value(X[m * K + k]) * inv"),
    ("bf16-round-truncating", "double sig = round_half_even(ldexp(a, 7 - E));",
     "double sig = floor(ldexp(a, 7 - E));"),
    ("bf16-subnormal-step", "round_half_even(ldexp(a, 133))", "round_half_even(ldexp(a, 134))"),
    ("bf16-overflow-threshold", "if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))",
     "if (a >= ldexp(2.0 - ldexp(1.0, -7), 127))"),
]

PIN_FUNCS = [getattr(m, n) for m in (pins, pins_i8, pins_ep, pins_norm) for n in dir(m) if n.startswith("test_")]


def _run_pins():
    """Names of pins that fail on the current library."""
    failed = []
    for f in PIN_FUNCS:
        if f.__name__ == "test_quantizer_worked_examples":
            cases = pins._load_worked()
            for c in cases:
                try:
                    f(c)
                except Exception:
                    failed.append(f.__name__ + "[" + c["name"] + "]")
            continue
        if hasattr(f, "pytestmark"):
            params = [m for m in f.pytestmark if m.name == "parametrize"]
            argnames, values = params[0].args
            argnames = [a.strip() for a in argnames.split(",")]
            for v in values:
                try:
                    f(**dict(zip(argnames, v)))
                except Exception:
                    failed.append(f.__name__)
            continue
        try:
            f()
        except Exception:
            failed.append(f.__name__)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique: " + name
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, "libmut.so")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                               "-shared", c, "-o", so, "-lm"])
        prev = oracle.use(oracle.open_lib(so))
        try:
            failed = _run_pins()
        finally:
            oracle.use(prev)
    assert failed, "no pin caught the planted mistake " + name
