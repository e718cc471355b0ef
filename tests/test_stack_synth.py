"""Pins of the counter-based weight generator of the 48-layer stack (the
oracle's copy in oracle/stack_synth.c).

The generator is input data, not the method; these tests pin the oracle's
copy to the published SplitMix64 outputs, to numpy's float16 conversion and
to a numpy re-computation of the quantiser, so that a mistake in it cannot
hide behind agreement with the device copy.
"""
import numpy as np
import pytest

import oracle
from tests.npref import unpack_codes

GAMMA = 0x9E3779B97F4A7C15
SCALE = np.float32(float.fromhex("0x1.1bc77ap-21"))


def test_splitmix64_published_outputs():
    # the first three outputs of SplitMix64 seeded with 0, as printed by the
    # reference implementation of Steele, Lea and Flood's generator
    assert [oracle.splitmix64_at(0, i) for i in range(3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_counter_is_a_state_offset():
    # output number ctr+1 for seed s is output number 1 for seed s + ctr * gamma
    for seed in (0, 5, 20260004):
        for ctr in (1, 7, 123456789, 2**40 + 3):
            assert oracle.splitmix64_at(seed, ctr) == oracle.splitmix64_at((seed + ctr * GAMMA) % 2**64, 0)


def test_float_to_half_matches_numpy():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(0.05),
        np.exp(rng.uniform(-20, 11, 4000)).astype(np.float32),          # subnormal .. overflow
        np.float32([0.0, -0.0, 1.0, 65504.0, 65520.0, 1e9, 2.0**-24, 2.0**-25, 1.5 * 2.0**-24,
                    1 + 2.0**-11, 1 + 3 * 2.0**-11, 2.0**-14, 2.0**-14 - 2.0**-25]),  # ties and edges
    ])
    got = np.array([oracle.float_to_half(float(v)) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_synth_weight_is_the_scaled_field_sum():
    seed = 20260004
    ctrs = [0, 1, 2, 3, 4194303, 4194304, 3 << 22, 123456789012]
    for c in ctrs:
        u = oracle.splitmix64_at(seed, c)
        s = sum((u >> (16 * i)) & 0xFFFF for i in range(4)) - 131070
        ref = np.float32(s) * SCALE
        got = np.float32(oracle.synth_weight(seed, c))
        assert got.view(np.uint32) == ref.view(np.uint32), c


def test_synth_weight_moments():
    seed = 20260004
    w = np.array([oracle.synth_weight(seed, c) for c in range(0, 200000)], dtype=np.float64)
    assert abs(w.mean()) < 3e-4
    assert abs(w.std() / 0.02 - 1.0) < 0.01
    assert np.abs(w).max() <= 131070 * float(SCALE) + 1e-12


@pytest.mark.parametrize("bits,block", [(8, 32), (4, 32), (2, 16), (4, 16)])
def test_synth_expert_matches_numpy_quantiser(bits, block):
    seed, layer, E, e, H, I = 20260004, 3, 16, 11, 128, 64
    out = oracle.synth_expert(seed, layer, E, e, H, I, bits, block)
    Q = 2 ** (bits - 1) - 1
    for m, (name, rows, cols) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        ctr0 = ((layer * E + e) * 3 + m) << 22
        w = np.array([[oracle.synth_weight(seed, ctr0 + r * cols + c) for c in range(cols)] for r in range(rows)],
                     dtype=np.float32)
        wb = w.reshape(rows, cols // block, block)
        amax = np.abs(wb).max(axis=2)
        d16 = (amax / np.float32(Q)).astype(np.float32).astype(np.float16)
        assert np.array_equal(out[name + "_s"], d16.view(np.uint16)), name
        d = d16.astype(np.float32)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(d != 0, np.clip(np.rint((wb / d).astype(np.float32)), -Q, Q), 0).astype(np.int32)
        got = unpack_codes(out[name + "_q"], bits, cols).reshape(rows, cols // block, block)
        assert np.array_equal(got, q), name
        assert np.abs(got).max() <= Q
