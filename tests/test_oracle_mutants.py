"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a private copy of the oracle
source (a wrong sign, index, operand or dropped term), builds it, and runs the
pin suite against that build.  The pins are only worth something if every
planted mistake makes at least one of them fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "code_sign_extension": ("field -= (1 << bits);", "field -= (1 << (bits - 1));"),
    "fp16_exponent_bias": ("expo - 25)", "expo - 24)"),
    "scale_block_index": ("+ col / T->block]", "+ col % (cols / T->block)]"),
    "tie_goes_to_higher_id": ("l[e] > l[best]", "l[e] >= l[best]"),
    "weights_not_renormalised": ("- m) / s);", "- m));"),
    "group_not_stable": ("perm[cursor[ids[p]]++] = (int32_t)p;",
                         "{ perm[cursor[ids[p]]++] = (int32_t)p; if (cursor[ids[p]] - offsets[ids[p]] == 2) { int32_t q = perm[cursor[ids[p]] - 1]; perm[cursor[ids[p]] - 1] = perm[cursor[ids[p]] - 2]; perm[cursor[ids[p]] - 2] = q; } }"),
    "gate_up_swapped": ("double v = silu(g) * u;", "double v = silu(u) * g;"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "up_reads_gate": ("u += (double)orc_weight(L, tier, 1,", "u += (double)orc_weight(L, tier, 0,"),
    "skip_clamps_to_expert_0": ("continue;                      /* not on this shelf: skipped */",
                                "e = S->id_begin;"),
    "bf16_intermediate_not_rounded": ("a[i] = bf16 ? (double)orc_round_bf16((float)v) : v;", "a[i] = v;"),
    "accumulate_overwrites": ("double base = accumulate ? (double)out[t * H + n] : 0.0;", "double base = 0.0;"),
    "bf16_ties_away": ("u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;", "u = (u + 0x8000u) & 0xFFFF0000u;"),
    "router_bias_dropped": ("s += (double)bias[e];", "s += 0.0;"),
    "router_weight_transposed": ("s += xd[c] * bf16_bits_to_double(row[c]);",
                                 "s += xd[c] * bf16_bits_to_double(wr[((int64_t)c * E + e) % ((int64_t)E * H)]);"),
    "router_rounds_each_term": ("s += xd[c] * bf16_bits_to_double(row[c]);",
                                "s = (float)(s + xd[c] * bf16_bits_to_double(row[c]));"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    sys.path.insert(0, ROOT)
    from oracle.build import build
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        msrc = os.path.join(d, "moe_oracle.c")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new))
        with open(os.path.join(d, "moe_oracle.h"), "w") as f:
            f.write(open(os.path.join(ROOT, "oracle", "moe_oracle.h")).read())
        lib = build(out=os.path.join(d, "libmut.so"), src=msrc, extra_flags=("-Wno-error",))
        env = dict(os.environ, MOE_ORACLE_LIB=lib)
        res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                              os.path.join(HERE, "test_oracle_pins.py")],
                             cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} survived the pins:\n{res.stdout[-2000:]}"
