"""Planted mistakes in the oracle (on the CPU) must each trip a pin.

Every mutant is a one-place textual change to moe_oracle.c of the kind a
careless implementation makes: a dropped term, a wrong sign, a wrong
index, a transposed operand, a wrong tie rule.  Each is compiled to a
temporary library and the pin suite is run against it in a subprocess
(so a crash also counts as caught).  The unmutated source must pass.

Not listed: dropping the -0 -> +0 canonicalisation of logits.  It is an
equivalent mutant -- float comparison already treats -0 and +0 as equal,
and an fp32 sum started from +0 never produces -0 -- so no pin can see it.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "tie_keeps_highest_index": ("l[e] > l[best]) best = e;", "l[e] >= l[best]) best = e;"),
    "bias_sign": ("if (bias) v = v + bias[e];", "if (bias) v = v - bias[e];"),
    "bias_dropped": ("if (bias) v = v + bias[e];", "if (bias) v = v;"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swapped": ("hid[i] = silu(g) * u;", "hid[i] = silu(u) * g;"),
    "no_renormalise": ("for (int r = 0; r < k; ++r) w[r] = w[r] / psum;", "for (int r = 0; r < k; ++r) w[r] = w[r];"),
    "softmax_no_max_shift_typo": ("z += exp((double)l[e] - m);\n    double psum", "z += exp((double)l[e]);\n    double psum"),
    "combine_wrong_rank": ("acc = acc + w[(size_t)t * k + j] * o[((size_t)t * k + j) * H + c];",
                           "acc = acc + w[(size_t)t * k + j] * o[((size_t)t * k + 0) * H + c];"),
    "combine_weight_misindexed": ("acc = acc + w[(size_t)t * k + j] * o[",
                                  "acc = acc + w[(size_t)t * k + (k - 1 - j)] * o["),
    "token_of_assignment": ("int t = a / k;", "int t = a % k;"),
    "shared_gate_dropped": ("if (I_s > 0) acc = acc + s[t] * os[(size_t)t * H + c];",
                            "if (I_s > 0) acc = acc + os[(size_t)t * H + c];"),
    "shared_gate_sign": ("s[t] = 1.0 / (1.0 + exp(-c));", "s[t] = 1.0 / (1.0 + exp(c));"),
    "down_transposed": ("acc += hid[i] * wmat_at(wd, row0 + (size_t)c, (size_t)i, I);",
                        "acc += hid[i] * wmat_at(wd, row0 + ((size_t)i * H + c) / I % H, ((size_t)i * H + c) % I, I);"),
    "e4m3_exponent_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e4m3_subnormal_as_normal": ("ldexp((double)m / 8.0, 1 - 7)", "ldexp(1.0 + (double)m / 8.0, 0 - 7)"),
    "e4m3_sign_dropped": ("return sgn ? -mag : mag;", "return mag;"),
    "fp8_scale_by_column": ("acc += (double)bf16_to_f32(x[i]) * (sc * m.q_val[q[i]]);",
                            "acc += (double)bf16_to_f32(x[i]) * ((double)m.scale[i % 8] * m.q_val[q[i]]);"),
    "fp8_down_scale_by_column": ("return (double)m.scale[r] * m.q_val", "return (double)m.scale[c] * m.q_val"),
    "q4_nibbles_swapped": ("int nib = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 15);",
                           "int nib = (c & 1) ? (row[c / 2] & 15) : (row[c / 2] >> 4);"),
    "q4_offset_binary": ("return nib >= 8 ? nib - 16 : nib;", "return nib - 8;"),
    "q4_group_of_scale": ("(f16_value(s[i / Q4_GROUP]) * (double)q4_weight(q, (size_t)i));",
                          "(f16_value(s[i % (n / Q4_GROUP)]) * (double)q4_weight(q, (size_t)i));"),
    "f16_exponent_bias": ("mag = ldexp(1.0 + (double)m / 1024.0, e - 15);", "mag = ldexp(1.0 + (double)m / 1024.0, e - 16);"),
    "align_not_stable": ("for (size_t a = 0; a < n; ++a) {\n        int e = ids[a];",
                         "for (size_t a = n; a-- > 0;) {\n        int e = ids[a];"),
    "ids_in_duplicates_accepted": ("if (ids_in[b] == ids_in[a]) { err = ORC_ERR_SHAPE; goto done; }",
                                   "if (ids_in[b] == ids_in[a] && 0) { err = ORC_ERR_SHAPE; goto done; }"),
    "ids_in_weights_from_own_selection": (
        "ids[(size_t)t * k + j] = e;\n                w[(size_t)t * k + j] = exp((double)l[e] - m) / z;",
        "w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - m) / z;\n"
        "                ids[(size_t)t * k + j] = e;"),
    "logit_dot_stride": ("float v = dot_bf16_f32(xt, w_router + (size_t)e * H, H);",
                         "float v = dot_bf16_f32(xt, w_router + (size_t)e, H - e);"),
}


def _compile(src_text, out):
    c = out + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    cmd = [a for a in oracle.GCC_CMD if a not in (oracle._SRC, oracle.LIB_PATH)]
    cmd = [x for x in cmd if x not in ("-o", "-lm")] + [c, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)


def _run_pins(lib):
    return subprocess.run([sys.executable, "-m", "tests.run_pins", lib], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


@pytest.fixture(scope="module")
def source():
    with open(oracle._SRC) as f:
        return f.read()


def test_unmutated_passes(source, tmp_path):
    lib = str(tmp_path / "orig.so")
    _compile(source, lib)
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(source, tmp_path, name):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} not found"
    lib = str(tmp_path / f"{name}.so")
    _compile(source.replace(old, new, 1), lib)
    r = _run_pins(lib)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout}{r.stderr}"
