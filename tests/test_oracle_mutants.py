"""Plant plausible mistakes in a copy of the oracle and check the pins see them.

Each mutant is a one-line change to ``oracle/moe_oracle.c`` (a swapped
operand, a wrong index, a dropped term, a wrong tie-break ...).  It is compiled
to a temporary library on the CPU, the pin tests run against it, and at least
one of them must fail.  The unmodified oracle passing the same pins is checked
by ``test_oracle_pins.py``.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

MUTANTS = {
    "gate_up_swapped": ("h[j] = silu(g) * u;", "h[j] = silu(u) * g;"),
    "down_transposed": ("acc += omat_at(D, n, j) * h[j];", "acc += omat_at(D, j % d, n % f) * h[j];"),
    "up_rows_offset": ("U->data = gu + f * d;\n        D->data = (const float*)",
                       "U->data = gu + (f - 1) * d;\n        D->data = (const float*)"),
    "ties_to_highest": ("if (best < 0 || logits[e] > logits[best]) best = e;",
                        "if (best < 0 || logits[e] >= logits[best]) best = e;"),
    "no_renormalisation": ("for (int j = 0; j < k; ++j) w[j] = p[sel[j]] / s;",
                           "for (int j = 0; j < k; ++j) w[j] = p[sel[j]];"),
    "sigmoid_router": ("p[e] = exp(logits[e] - mx);", "p[e] = 1.0 / (1.0 + exp(-logits[e]));"),
    "bias_dropped": ("logits[e] = acc + (bias ? (double)bias[e] : 0.0);", "logits[e] = acc;"),
    "bias_sign": ("logits[e] = acc + (bias ? (double)bias[e] : 0.0);",
                  "logits[e] = acc - (bias ? (double)bias[e] : 0.0);"),
    "shared_dropped": ("for (long n = 0; n < d; ++n) acc[n] += y[n];", ";"),
    "routed_unweighted": ("acc[n] += wj * y[n];", "acc[n] += y[n];"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "router_transposed": ("acc += x[i] * (double)Wr[(long)e * d + i];",
                          "acc += x[i] * (double)Wr[((long)i * E + e) % ((long)E * d)];"),
    "nibble_order": ("(c % 2 == 0) ? (byte & 0xF) : (byte >> 4)",
                     "(c % 2 == 1) ? (byte & 0xF) : (byte >> 4)"),
    "block_scale_index": ("uint8_t sc = m->scales[r * (m->cols / 16) + c / 16];",
                          "uint8_t sc = m->scales[r * (m->cols / 16) + (c / 16 + 1) % (m->cols / 16)];"),
    "tensor_scale_swap": ("G->tensor_scale = (double)tscales[3 * e + 0];",
                          "G->tensor_scale = (double)tscales[3 * e + 1];"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e4m3_bias": ("v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    "bf16_mantissa": ("v = ldexp(1.0 + m / 128.0, e - 127);", "v = ldexp(1.0 + m / 256.0, e - 127);"),
    "rmsnorm_no_mean": ("double r = 1.0 / sqrt(ss / d + eps);", "double r = 1.0 / sqrt(ss + eps);"),
    "round_ties_up": ("double r = nearbyint(ldexp(a, 7 - e));", "double r = floor(ldexp(a, 7 - e) + 0.5);"),
}

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _build(src_text, tmpdir, name):
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as fh:
        fh.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-w", "-o", so, c, "-lm"], check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor must occur exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        so = _build(text.replace(old, new), tmp, name)
        failed = []
        with oracle.using_library(so):
            for pin in PINS:
                try:
                    pin()
                except (AssertionError, ValueError):
                    failed.append(pin.__name__)
        assert failed, "no pin noticed the planted mistake %r" % name
