"""The oracle against its pins, and planted mistakes in the oracle against
the same pins (each must be caught by at least one)."""
import os
import shutil

import pytest

import oracle
import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# (name, text in oracle.c, replacement): plausible slips in the arithmetic
MUTANTS = [
    ("causal edge off by one", "(j <= i)", "(j < i)"),
    ("window edge off by one", "i - j < (int64_t)window", "i - j <= (int64_t)window"),
    ("span end inclusive", "j < span_hi", "j <= span_hi"),
    ("span start exclusive", "j >= span_lo", "j > span_lo"),
    ("no max subtraction", "s[a] = exp(s[a] - m);", "s[a] = exp(s[a]);"),
    ("wrong GQA head map", "int32_t g = h / group;", "int32_t g = h % hkv;"),
    ("decode GQA head map", "g = h / group;\n", "g = h % hkv;\n"),
    ("decode slot index", "int64_t slot = j % block_size;", "int64_t slot = (j + 1) % block_size;"),
    ("V read with K operand", "out[c] += p * load_elem(v,", "out[c] += p * load_elem(k,"),
    ("scale dropped", "s[a] = scale * dot;", "s[a] = dot;"),
    ("first weight dropped from Z", "z += s[a];", "if (a) z += s[a];"),
    ("lse misses max", "*lse = m + log(z);", "*lse = log(z);"),
    ("decode window ignored", "if (!allowed(i, j, window, -1, -1)) continue;",
     "if (!allowed(i, j, -1, -1, -1)) continue;"),
    ("transposed query/key offset", "load_elem(q, qt, q_off + c) * load_elem(k, kvt, key_off[a] + c)",
     "load_elem(q, qt, q_off + c) * load_elem(k, kvt, key_off[n - 1 - a] + c)"),
    ("bf16 widening without the shift", "[idx]) << 16;", "[idx]);"),
    ("bf16 widening shifted by 15", "[idx]) << 16;", "[idx]) << 15;"),
    ("bf16 element index off", "((const uint16_t*)base)[idx])", "((const uint16_t*)base)[idx ^ 1])"),
    ("fp32 element index off", "((const float*)base)[idx];", "((const float*)base)[idx ^ 1];"),
    ("fp32 read as bf16", "if (dtype == ORACLE_F32)", "if (dtype == -5)"),
    ("backward units: statistics of one head per group",
     "h < (g + 1) * group; ++h)\n                    need[", "h < g * group + 1; ++h)\n                    need["),
    ("backward: ds sign", "double ds = p * (dp - del);", "double ds = p * (del - dp);"),
    ("backward: dk misses scale", "dkj[c] += scale * ds *", "dkj[c] += ds *"),
    ("backward: dv uses ds", "dvj[c] += p * load_elem(dout", "dvj[c] += ds * load_elem(dout"),
    ("backward: delta from v", "del += load_elem(dout, dodtype, w * (int64_t)d + c) * o[c];",
     "del += load_elem(dout, dodtype, w * (int64_t)d + c) * load_elem(v, kvdtype, c);"),
    ("backward: dq uses q", "dqi[c] += scale * ds * load_elem(k, kvdtype, key_off[a] + c);",
     "dqi[c] += scale * ds * load_elem(q, qdtype, w * (int64_t)d + c);"),
    ("prologue: rope partner", "const double a = y[i], b = y[i + half];",
     "const double a = y[i], b = y[half - 1 - i + half];"),
    ("prologue: rope sign", "y[i] = a * c - b * s;", "y[i] = a * c + b * s;"),
    ("prologue: frequency exponent", "pow(theta, -2.0 * i / freq_dims)",
     "pow(theta, -1.0 * i / freq_dims)"),
    ("prologue: mean over d - 1", "sqrt(ss / d + eps)", "sqrt(ss / (d - 1) + eps)"),
    ("prologue: eps outside the root", "1.0 / sqrt(ss / d + eps)", "1.0 / (sqrt(ss / d) + eps)"),
    ("prologue: offset ignored", "(offset + load_elem(weight, wdtype, j))",
     "(load_elem(weight, wdtype, j))"),
    ("prologue: position of another row", "const int64_t row = rh / heads;",
     "const int64_t row = rh % heads;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = oracle.build(src=str(mutated), out=str(tmp_path / "liboracle_mutant.so"), werror=False)
    lib = oracle.open_library(so)
    # the pins of the mutated function's own family first; stop at the first catch
    family = name.split(":")[0] if ":" in name else ""
    pins = sorted(oracle_pins.ALL_PINS, key=lambda f: 0 if family and family in f.__name__ else 1)
    caught = []
    for pin in pins:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name!r}"
