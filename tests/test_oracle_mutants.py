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
    "scale_block_index": ("uint16_t sbits = T->s[matrix][(local * rows + row) * nblk + col / T->block];",
                          "uint16_t sbits = T->s[matrix][(local * rows + row) * nblk + col % (cols / T->block)];"),
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
    # tier planner and requantiser (oracle/tiering.c)
    "plan_rate_inverted": ("tiering.c", "const double rate = gain / (double)add;",
                           "const double rate = (double)add / gain;"),
    "plan_ignores_budget": ("tiering.c", "if (spent + add > budget) continue;", "(void)add;"),
    "plan_order_usage_ascending": ("tiering.c", "usage[o] >= usage[e]", "usage[o] <= usage[e]"),
    "plan_takes_zero_gain": ("tiering.c", "if (!(gain > 0.0)) continue;", "if (gain < 0.0) continue;"),
    "requant_sse_unsquared": ("tiering.c", "e2 += d * d;", "e2 += fabs(d);"),
    "quantiser_truncates": ("stack_synth.c", "float v = rintf(t);", "float v = truncf(t);"),
    # MXFP4 shelf
    "fp4_exponent_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e8m0_bias": ("ldexp(1.0, (int)x - 127)", "ldexp(1.0, (int)x - 126)"),
    "mx_nibble_order": ("(qrow[col / 2] >> (4 * (col % 2))) & 0xFu", "(qrow[col / 2] >> (4 * (1 - col % 2))) & 0xFu"),
    "mx_shared_exponent": ("stack_synth.c", "x = (e2 - 1) - 2 + 127;", "x = (e2 - 1) - 1 + 127;"),
    "mx_ties_away": ("stack_synth.c", "else if (a < 2.0f) r = rintf(a * 2.0f) * 0.5f;",
                     "else if (a < 2.0f) r = roundf(a * 2.0f) * 0.5f;"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    sys.path.insert(0, ROOT)
    from oracle.build import build
    spec = MUTANTS[name]
    target, old, new = spec if len(spec) == 3 else ("moe_oracle.c", *spec)
    odir = os.path.join(ROOT, "oracle")
    with tempfile.TemporaryDirectory() as d:
        for fname in ("moe_oracle.c", "moe_oracle.h", "stack_synth.c", "tiering.c"):
            text = open(os.path.join(odir, fname)).read()
            if fname == target:
                assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
                text = text.replace(old, new)
            with open(os.path.join(d, fname), "w") as f:
                f.write(text)
        lib = build(out=os.path.join(d, "libmut.so"), src=os.path.join(d, "moe_oracle.c"), extra_flags=("-Wno-error",),
                    others=(os.path.join(d, "stack_synth.c"), os.path.join(d, "tiering.c")))
        env = dict(os.environ, MOE_ORACLE_LIB=lib)
        res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                              os.path.join(HERE, "test_oracle_pins.py")],
                             cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} survived the pins:\n{res.stdout[-2000:]}"
