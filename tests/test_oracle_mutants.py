"""Every plausible mistake planted in a copy of the oracle trips a pin.

Each mutant is the oracle's source with one textual change (a dropped term,
a wrong sign, index or operand, a swapped field), compiled into a temporary
directory on the CPU and run through all pins in a child process.  A mutant
that no pin catches means the pins leave that part of the oracle unchecked.
"""
import concurrent.futures as cf
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "bit_order_reversed": [("return (int)((word >> (bit % 32)) & ((1u << bits) - 1u));",
                            "return (int)((word >> (32 - bits - bit % 32)) & ((1u << bits) - 1u));")],
    "code_mask_always_4bit": [("return (int)((word >> (bit % 32)) & ((1u << bits) - 1u));",
                               "return (int)((word >> (bit % 32)) & 0xFu);")],
    "scale_bias_halves_swapped": [("*scale = bf16_to_double(word & 0xFFFFu);", "*scale = bf16_to_double(word >> 16);"),
                                  ("*bias = bf16_to_double(word >> 16);", "*bias = bf16_to_double(word & 0xFFFFu);")],
    "bias_sign": [("return (double)orc_q(blob, D, I, bits, mat, row, col) * s + b;",
                   "return (double)orc_q(blob, D, I, bits, mat, row, col) * s - b;")],
    "down_uses_up_scales": [("(uint64_t)mat * (elems / (uint64_t)group) * 4",
                             "(uint64_t)(mat == 2 ? 1 : mat) * (elems / (uint64_t)group) * 4")],
    "group_of_32": [("(uint64_t)(col / group);", "(uint64_t)(col / group / 2);")],
    "bf16_shift": [("uint32_t u = h16 << 16;", "uint32_t u = h16 << 15;")],
    "fma_form_drops_x_in_bias": [("fma(q, s * x[j], b * x[j])", "fma(q, s * x[j], b)")],
    "group_form_drops_sum_x": [("acc += s * qx + b * xs;", "acc += s * qx + b;")],
    "router_transposed": [("Wr[(size_t)e * (size_t)D + (size_t)d]", "Wr[(size_t)d * (size_t)E + (size_t)e]")],
    "ties_to_higher_index": [("logits[e] > logits[best])) best = e;", "logits[e] >= logits[best])) best = e;")],
    "gap_from_top1": [("*gap = (K < E) ? logits[sel[K - 1]] - next : INFINITY;",
                       "*gap = (K < E) ? logits[sel[0]] - next : INFINITY;")],
    "softmax_sign": [("for (int k = 0; k < K; ++k) w[k] = exp(logits[sel[k]] - m) / z;",
                      "for (int k = 0; k < K; ++k) w[k] = exp(m - logits[sel[k]]) / z;")],
    "uniform_weights": [("for (int k = 0; k < K; ++k) w[k] = exp(logits[sel[k]] - m) / z;",
                         "for (int k = 0; k < K; ++k) w[k] = 1.0 / K;")],
    "silu_sign": [("hh[i] = g / (1.0 + exp(-g)) * u;", "hh[i] = g / (1.0 + exp(g)) * u;")],
    "gate_up_swapped": [("hh[i] = g / (1.0 + exp(-g)) * u;", "hh[i] = u / (1.0 + exp(-u)) * g;")],
    "gate_reads_up": [("g += orc_w(blob, D, I, bits, group, 0, i, j) * x[j];",
                       "g += orc_w(blob, D, I, bits, group, 1, i, j) * x[j];")],
    "shared_dropped": [("for (int o = 0; o < D; ++o) c[o] += y[o];", "for (int o = 0; o < D; ++o) c[o] += 0.0 * y[o];")],
    "shared_gated_by_w0": [("for (int o = 0; o < D; ++o) c[o] += y[o];", "for (int o = 0; o < D; ++o) c[o] += w[0] * y[o];")],
    "combine_wrong_slot_weight": [("for (int o = 0; o < D; ++o) c[o] += w[k] * y[o];",
                                   "for (int o = 0; o < D; ++o) c[o] += w[0] * y[o];")],
    "residual_dropped": [("r_out[o] = r[o] + c[o];", "r_out[o] = c[o];")],
    "eps_outside_sqrt": [("double inv = 1.0 / sqrt(ss / (double)D + eps);",
                          "double inv = 1.0 / (sqrt(ss / (double)D) + eps);")],
    "mean_over_D_minus_1": [("double inv = 1.0 / sqrt(ss / (double)D + eps);",
                             "double inv = 1.0 / sqrt(ss / (double)(D - 1) + eps);")],
    "gamma_dropped": [("x_out[o] = r_out[o] * inv * (double)gamma[o];", "x_out[o] = r_out[o] * inv;")],
    "group_offset_not_cumulative": [("offset[e + 1] = offset[e] + n;", "offset[e + 1] = n;")],
}

_RUNNER = r"""
import json, sys
sys.path[:0] = [sys.argv[2], sys.argv[2] + '/tests']
import oracle, oracle_pins
L = oracle.load(sys.argv[1])
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(L)
    except Exception as e:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""


def _run_mutant(name, edits, tmpdir):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"{name}: pattern not unique in oracle.c: {old!r}"
        src = src.replace(old, new)
    d = os.path.join(tmpdir, name)
    os.makedirs(d, exist_ok=True)
    for f in ("oracle.h",):
        with open(os.path.join(ROOT, "oracle", f)) as fi, open(os.path.join(d, f), "w") as fo:
            fo.write(fi.read())
    c = os.path.join(d, "oracle.c")
    with open(c, "w") as f:
        f.write(src)
    so = os.path.join(d, "liboracle_mut.so")
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99", c,
                           "-o", so, "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-c", _RUNNER, so, ROOT], capture_output=True, text=True, timeout=300,
                       env=env)
    if p.returncode != 0:
        return ["<crashed>"]
    return json.loads(p.stdout.strip().splitlines()[-1])


def test_every_mutant_is_caught(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_mutant, name, edits, str(tmp_path)) for name, edits in MUTANTS.items()}
        results = {name: f.result() for name, f in futs.items()}
    survivors = [n for n, failed in results.items() if not failed]
    assert not survivors, f"mutants no pin catches: {survivors}"
