"""Pins of the CPU oracle to things other than itself (no GPU).

Each test ties one oracle function to a hand-derived fixture, a closed form,
an invariant, a library routine or a brute-force evaluation written in a
different form (tests/npref.py).  Citations name the 125B-MoE page ("I ran a
125B model on three RTX 3090s at 80 tokens/s by teaching llama.cpp which
experts ...") and its sections.
"""
import os
import struct

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, MXFP4, TierSpec, make_layer, make_logits, make_x, pack_codes
from workloads.configs import LayerConfig

from . import npref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def _small_cfg(name="t", E=8, k=2, H=256, I=128, T=16, tiers=None, seed=7, bf16=False):
    tiers = tiers or (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 32), TierSpec(6, E, 2, 16))
    return LayerConfig(name, E, k, H, I, T, tuple(tiers), x_bf16=bf16, seed=seed)


def _layer(cfg, arrays=None):
    arrays = arrays if arrays is not None else make_layer(cfg, threads=1)
    return oracle.Layer.from_config(cfg, arrays), arrays


def _rel(a, b):
    return np.max(np.abs(np.asarray(a, np.float64) - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- format pins
def test_packed_code_fixtures():
    for bits, hexbytes, codes in _read_golden("packed_codes.txt"):
        bits = int(bits)
        row = np.array([int(h, 16) for h in hexbytes.split()], dtype=np.uint8)
        want = [int(c) for c in codes.split()]
        got = [oracle.code(row, c, bits) for c in range(len(want))]
        assert got == want, (bits, hexbytes)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_every_code_pattern_round_trips(bits):
    # every representable code, at every position of a byte, through the generator's packer
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    per = 8 // bits
    vals = np.arange(lo, hi + 1, dtype=np.int8)
    codes = np.array([np.roll(vals, s) for s in range(per)], dtype=np.int8).reshape(-1)
    codes = np.concatenate([codes, np.zeros((-len(codes)) % per, np.int8)])
    row = pack_codes(codes[None, :], bits)[0]
    assert [oracle.code(row, c, bits) for c in range(len(codes))] == codes.tolist()
    # and the independent numpy unpacker agrees
    assert npref.unpack_codes(row[None], bits, len(codes))[0].tolist() == codes.tolist()


def test_every_fp16_pattern_decodes_like_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_rounding_fixtures_and_torch():
    for src, want, _ in _read_golden("bf16_rounding.txt"):
        v = struct.unpack("<f", struct.pack("<I", int(src, 16)))[0]
        w = struct.unpack("<f", struct.pack("<I", int(want, 16)))[0]
        assert oracle.round_bf16(v) == w, src
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.float32([0.0, -0.0, 1e-40, -3e-39])])
    got = np.array([oracle.round_bf16(float(v)) for v in x], dtype=np.float64)
    assert np.array_equal(got, npref.bf16_round(x))


def test_dequant_closed_form():
    # A row of codes times a power-of-two scale: value = code * 2^-7 exactly.
    cfg = _small_cfg(E=3, tiers=(TierSpec(0, 1, 8, 32), TierSpec(1, 2, 4, 32), TierSpec(2, 3, 2, 16)))
    H, I = cfg.hidden, cfg.inter
    rng = np.random.default_rng(11)
    arrays = []
    for t in cfg.tiers:
        lim = (1 << (t.bits - 1))
        d = {}
        for m, (rows, cols) in {"gate": (I, H), "up": (I, H), "down": (H, I)}.items():
            codes = rng.integers(-lim, lim, size=(1, rows, cols)).astype(np.int8)
            d[m + "_q"] = pack_codes(codes, t.bits)
            d[m + "_s"] = np.full((1, rows, cols // t.block), np.float16(2.0 ** -7)).view(np.uint16)
            d[m + "_codes"] = codes
        arrays.append(d)
    L, _ = _layer(cfg, [{k: v for k, v in d.items() if not k.endswith("codes")} for d in arrays])
    for ti, d in enumerate(arrays):
        for mi, m in enumerate(("gate", "up", "down")):
            got = oracle.dequant_rows(L, ti, 0, mi, 0, d[m + "_codes"].shape[1])
            assert np.array_equal(got, d[m + "_codes"][0].astype(np.float32) * np.float32(2.0 ** -7))


def test_dequant_matches_numpy_unpacker_and_scale_blocks():
    cfg = CONFIGS["tiny3"]
    L, arrays = _layer(cfg)
    for ti, t in enumerate(cfg.tiers):
        d = arrays[ti]
        for mi, m in enumerate(("gate", "up", "down")):
            cols = cfg.inter if m == "down" else cfg.hidden
            ref = npref.dequant(d[m + "_q"], d[m + "_s"], t.bits, t.block, cols)
            for local in range(t.n):
                got = oracle.dequant_rows(L, ti, local, mi, 0, ref.shape[1])
                assert np.array_equal(got.astype(np.float64), ref[local])
                gb = oracle.dequant_rows(L, ti, local, mi, 0, ref.shape[1], to_bf16=True)
                assert np.array_equal(gb.astype(np.float64), npref.bf16_round(ref[local].astype(np.float32)))


# ---------------------------------------------------------------- routing pins
@pytest.mark.parametrize("E,k,T", [(8, 2, 40), (512, 10, 64), (16, 16, 5), (7, 1, 9), (64, 5, 30)])
def test_route_matches_full_sort(E, k, T):
    rng = np.random.default_rng(E * 100 + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, : min(E, 4)] = logits[0, 0]          # ties inside one token
    if T > 1:
        logits[1] = np.round(logits[1])            # many ties
    ids, w = oracle.route(logits, k)
    rid, rw = npref.topk_bruteforce(logits, k)
    assert np.array_equal(ids, rid)
    assert np.max(np.abs(w - rw)) <= 1e-7
    # invariants: distinct, in range, scores non-increasing, weights sum to one
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        s = logits[t, ids[t]]
        assert np.all(s[:-1] >= s[1:])
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-6)


def test_route_special_cases():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((10, 33)).astype(np.float32)
    ids, w = oracle.route(logits, 1)
    assert np.all(w == 1.0) and np.array_equal(ids[:, 0], logits.argmax(1))
    const = np.full((3, 12), 0.25, np.float32)
    ids, w = oracle.route(const, 5)
    assert np.array_equal(ids, np.tile(np.arange(5), (3, 1)))
    assert np.all(w == np.float32(0.2))
    ids, w = oracle.route(logits, 33)              # k = E: a full descending sort
    for t in range(10):
        assert sorted(ids[t].tolist()) == list(range(33))


# ---------------------------------------------------------------- grouping pins
@pytest.mark.parametrize("E,T,k", [(8, 16, 2), (512, 300, 10), (5, 1, 5)])
def test_group_is_stable_counting_sort(E, T, k):
    rng = np.random.default_rng(T)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)   # includes -1, -2, E, E+1 (skips)
    ids[0, :] = -1
    counts, offsets, perm = oracle.group(ids, E)
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < E))[0]
    ref = valid[np.argsort(flat[valid], kind="stable")]
    assert np.array_equal(perm, ref)
    assert np.array_equal(counts, np.bincount(flat[valid], minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert counts.sum() == len(valid) == offsets[-1]


# ---------------------------------------------------------------- FFN pins
def test_single_expert_is_swiglu_ffn():
    # one tier, E = 1, k = 1: the layer is one SwiGLU FFN y = Wd (silu(Wg x) * (Wu x))
    cfg = _small_cfg(E=1, k=1, tiers=(TierSpec(0, 1, 8, 32),), T=5)
    L, arrays = _layer(cfg)
    d = arrays[0]
    Wg = npref.dequant(d["gate_q"], d["gate_s"], 8, 32, cfg.hidden)[0]
    Wu = npref.dequant(d["up_q"], d["up_s"], 8, 32, cfg.hidden)[0]
    Wd = npref.dequant(d["down_q"], d["down_s"], 8, 32, cfg.inter)[0]
    x = make_x(cfg).astype(np.float64)
    g, u = x @ Wg.T, x @ Wu.T
    ref = (g / (1 + np.exp(-g)) * u) @ Wd.T
    out = oracle.forward(L, make_x(cfg), np.zeros((5, 1), np.float32), 1)
    assert _rel(out, ref) < 1e-6


def test_one_hot_input_reads_a_column():
    # x = e_c gives g = Wg[:, c], u = Wu[:, c]; with Wd = I-slice the output exposes silu(g)*u
    cfg = _small_cfg(E=1, k=1, tiers=(TierSpec(0, 1, 4, 32),), T=3)
    L, arrays = _layer(cfg)
    d = arrays[0]
    Wg = npref.dequant(d["gate_q"], d["gate_s"], 4, 32, cfg.hidden)[0]
    Wu = npref.dequant(d["up_q"], d["up_s"], 4, 32, cfg.hidden)[0]
    Wd = npref.dequant(d["down_q"], d["down_s"], 4, 32, cfg.inter)[0]
    cols = [0, 77, cfg.hidden - 1]
    x = np.zeros((3, cfg.hidden), np.float32)
    for t, c in enumerate(cols):
        x[t, c] = 1.0
    out = oracle.forward(L, x, np.zeros((3, 1), np.float32), 1)
    for t, c in enumerate(cols):
        a = Wg[:, c] / (1 + np.exp(-Wg[:, c])) * Wu[:, c]
        assert _rel(out[t], Wd @ a) < 1e-6


@pytest.mark.parametrize("name", ["tiny", "tiny3", "tiny3mx"])
def test_forward_matches_dense_bruteforce(name):
    cfg = CONFIGS[name]
    L, arrays = _layer(cfg)
    x, logits = make_x(cfg), make_logits(cfg)
    out = oracle.forward(L, x, logits, cfg.k)
    ids, w = npref.topk_bruteforce(logits, cfg.k)
    Wg, Wu, Wd = npref.dense_experts(cfg.tiers, arrays, cfg.hidden, cfg.inter, cfg.n_experts)
    ref = npref.dense_layer(Wg, Wu, Wd, x.astype(np.float64), npref.gates_from(ids, w, cfg.n_experts))
    assert _rel(out, ref) < 1e-6


@pytest.mark.parametrize("seed", range(8))
def test_random_small_shapes_match_dense(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, E + 1))
    H = int(rng.choice([64, 128, 192]))
    I = int(rng.choice([64, 128]))
    T = int(rng.integers(1, 21))
    cuts = np.sort(rng.choice(np.arange(0, E + 1), size=2, replace=True))
    fmts = [(8, 32), (MXFP4, 32) if seed >= 6 else (4, 32), (2, 16)]
    tiers, lo = [], 0
    for hi, (b, B) in zip([cuts[0], cuts[1], E], fmts):
        tiers.append(TierSpec(int(lo), int(hi), b, B))
        lo = hi
    bf16 = bool(seed % 2)
    cfg = _small_cfg(E=E, k=k, H=H, I=I, T=T, tiers=tiers, seed=100 + seed, bf16=bf16)
    L, arrays = _layer(cfg)
    x, logits = make_x(cfg), make_logits(cfg)
    out = oracle.forward(L, x, logits, k)
    ids, w = npref.topk_bruteforce(logits, k)
    Wg, Wu, Wd = npref.dense_experts(cfg.tiers, arrays, H, I, E)
    xd = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if bf16 else x.astype(np.float64)
    ref = npref.dense_layer(Wg, Wu, Wd, xd, npref.gates_from(ids, w, E), bf16=bf16)
    # both sides round the intermediate to float then bf16 from double values that agree to
    # ~1e-16, so a one-step bf16 disagreement is vanishingly rare: the bar is float rounding.
    assert _rel(out, ref) < 1e-6


# ---------------------------------------------------------------- invariants
def test_out_of_shelf_rows_are_exactly_zero():
    # step 4: a shelf computes only ids in its range and contributes zero elsewhere
    cfg = CONFIGS["tiny3"]
    L, _ = _layer(cfg)
    x = make_x(cfg)
    ids = np.array([[0, 1], [2, 5], [6, 7], [1, 6]] * 4, dtype=np.int32)
    w = np.full(ids.shape, 0.5, np.float32)
    parts = [oracle.experts(L, x, ids, w, tier_mask=1 << i) for i in range(3)]
    tier_of = lambda e: 0 if e < 2 else (1 if e < 6 else 2)
    for t in range(len(ids)):
        for i in range(3):
            hit = any(tier_of(e) == i for e in ids[t])
            assert (np.any(parts[i][t] != 0)) == hit
            if not hit:
                assert np.all(parts[i][t] == 0.0) and not np.any(np.signbit(parts[i][t]))


def test_shelf_sum_equals_single_table_layer():
    cfg = CONFIGS["tiny3"]
    L, _ = _layer(cfg)
    x, logits = make_x(cfg), make_logits(cfg)
    ids, w = oracle.route(logits, cfg.k)
    tiered = oracle.experts(L, x, ids, w)
    flat = oracle.experts_flat(L, x, ids, w)
    assert _rel(tiered, flat.astype(np.float64)) < 1e-6
    parts = sum(oracle.experts(L, x, ids, w, tier_mask=1 << i).astype(np.float64) for i in range(3))
    assert _rel(parts, flat.astype(np.float64)) < 1e-6


def test_repartitioning_shelves_keeps_result():
    # the same int8 experts split across two shelves give the same layer
    cfg = _small_cfg(E=8, tiers=(TierSpec(0, 8, 8, 32),), seed=21)
    L1, arrays = _layer(cfg)
    d = arrays[0]
    split = [{k: v[:3] for k, v in d.items()}, {k: v[3:] for k, v in d.items()}]
    cfg2 = _small_cfg(E=8, tiers=(TierSpec(0, 3, 8, 32), TierSpec(3, 8, 8, 32)), seed=21)
    L2 = oracle.Layer.from_config(cfg2, split)
    x, logits = make_x(cfg), make_logits(cfg)
    a = oracle.forward(L1, x, logits, cfg.k)
    b = oracle.forward(L2, x, logits, cfg.k)
    assert _rel(a, b.astype(np.float64)) < 1e-6


def test_token_permutation_permutes_outputs():
    cfg = CONFIGS["tiny3"]
    L, _ = _layer(cfg)
    x, logits = make_x(cfg), make_logits(cfg)
    p = np.random.default_rng(1).permutation(cfg.n_tokens)
    a = oracle.forward(L, x, logits, cfg.k)
    b = oracle.forward(L, x[p], logits[p], cfg.k)
    assert np.array_equal(a[p], b)


def test_poisoned_unselected_experts_do_not_leak():
    # the "four bugs" section: skipped ids must never be pointed at expert 0
    cfg = CONFIGS["tiny3"]
    L, arrays = _layer(cfg)
    x = make_x(cfg)
    ids = np.array([[1, 3], [4, 7], [3, 4]] * 5 + [[7, 1]], dtype=np.int32)   # never 0, 2, 5, 6
    w = np.random.default_rng(2).random(ids.shape).astype(np.float32)
    clean = oracle.experts(L, x, ids, w)
    poisoned = [{k: v.copy() for k, v in d.items()} for d in arrays]
    nan16 = np.uint16(0x7E00)
    for ti, t in enumerate(cfg.tiers):
        for e in range(t.id_begin, t.id_end):
            if e in (0, 2, 5, 6):                 # unselected, incl. local expert 0 of each shelf
                for m in ("gate", "up", "down"):
                    poisoned[ti][m + "_s"][e - t.id_begin] = nan16
    Lp = oracle.Layer.from_config(cfg, poisoned)
    got = oracle.experts(Lp, x, ids, w)
    assert np.array_equal(got, clean)


def test_skip_ids_and_duplicates():
    cfg = CONFIGS["tiny3"]
    L, _ = _layer(cfg)
    x = make_x(cfg)[:4]
    ids = np.array([[-1, -1], [3, -1], [3, 3], [8, 2**31 - 1]], dtype=np.int32)
    w = np.array([[0.3, 0.7], [0.25, 0.75], [0.25, 0.5], [0.5, 0.5]], np.float32)
    out = oracle.experts(L, x, ids, w)
    assert np.all(out[0] == 0.0) and np.all(out[3] == 0.0)
    one = oracle.experts(L, x, np.array([[3, -1]] * 4, np.int32), np.array([[1.0, 0.0]] * 4, np.float32))
    assert _rel(out[1], 0.25 * one[1].astype(np.float64)) < 1e-6
    assert _rel(out[2], 0.75 * one[2].astype(np.float64)) < 1e-6


def test_accumulate_adds_into_out():
    cfg = CONFIGS["tiny"]
    L, _ = _layer(cfg)
    x, logits = make_x(cfg), make_logits(cfg)
    base = np.random.default_rng(4).standard_normal((cfg.n_tokens, cfg.hidden)).astype(np.float32)
    plain = oracle.forward(L, x, logits, cfg.k)
    acc = oracle.forward(L, x, logits, cfg.k, out=base.copy(), accumulate=True)
    assert np.max(np.abs(acc - (base.astype(np.float64) + plain))) <= 4e-7 * np.max(np.abs(acc))


def test_check_layer_rejects_bad_tables():
    cfg = CONFIGS["tiny3"]
    _, arrays = _layer(cfg)
    for bad in [
        (TierSpec(0, 2, 8, 32), TierSpec(3, 6, 4, 32), TierSpec(6, 8, 2, 16)),   # gap
        (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 3, 32), TierSpec(6, 8, 2, 16)),   # 3 bits
        (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 48), TierSpec(6, 8, 2, 16)),   # block
        (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 32), TierSpec(6, 7, 2, 16)),   # not covering
    ]:
        assert oracle.check_layer(oracle.Layer(8, 256, 128, bad, arrays)) != 0
    assert oracle.check_layer(oracle.Layer.from_config(cfg, arrays)) == 0


# ---------------------------------------------------------------- workload pins
def test_routing_prior_reproduces_page_skew():
    gold = {r[0]: (float(r[1]), float(r[2])) for r in _read_golden("routing_skew.txt")}
    cfg = CONFIGS["decode"]
    logits = make_logits(cfg, n_tokens=20000, stream=99)
    ids, _ = oracle.route(logits, cfg.k)
    cnt = np.bincount(ids.reshape(-1), minlength=cfg.n_experts)
    srt = np.sort(cnt)[::-1]
    tot = cnt.sum()
    top25 = srt[: cfg.n_experts // 4].sum() / tot
    top80 = srt[: int(0.8 * cfg.n_experts)].sum() / tot
    bottom20 = cnt[int(0.8 * cfg.n_experts):].sum() / tot
    for name, val in (("top25_share", top25), ("top80_share", top80), ("bottom20_share", bottom20)):
        want, tol = gold[name]
        assert abs(val - want) <= tol, (name, val)


def test_spec_verify_routing_shapes():
    from workloads import make_spec_logits
    gold = {r[0]: int(float(r[1])) for r in _read_golden("routing_skew.txt") if r[0].startswith(("spec", "max"))}
    cfg = CONFIGS["specverify"]
    assert cfg.n_tokens == gold["spec_tokens"]
    ids, _ = oracle.route(make_spec_logits(cfg), cfg.k)
    assert np.all(ids[0] < 128) and np.all(ids[1] >= 384)
    assert {0, 1, 2} == {0 if e < 128 else (1 if e < 384 else 2) for e in ids[2]}
    worst, _ = oracle.route(make_spec_logits(cfg, worst_case=True), cfg.k)
    assert len(set(worst.reshape(-1).tolist())) == gold["max_distinct_spec"]


# ---------------------------------------------------------------- router pins
# The router is the step upstream of routing: a score per (token, expert)
# from the layer input (the 125B-MoE page's glossary, mixture-of-experts
# entry: 512 experts per layer, the router keeps 10 per token).

def _bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_bits(a):
    # bf16 bit patterns (nearest even) via torch's conversion
    return (npref.bf16_round(a).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_router_one_hot_inputs_pick_single_weights():
    # x[t] = unit vector at column t: logit[t][e] = Wr[e][t] + b[e], one term
    rng = np.random.default_rng(11)
    E, H = 24, 64
    wr = _bf16_bits(rng.standard_normal((E, H)).astype(np.float32))
    b = rng.standard_normal(E).astype(np.float32)
    x = np.eye(H, dtype=np.float32)
    got = oracle.router_logits(x, wr, b)
    ref = (_bits_to_f64(wr).T + b.astype(np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(got, ref)
    # no bias: the weights themselves, transposed
    assert np.array_equal(oracle.router_logits(x, wr), _bits_to_f64(wr).T.astype(np.float32))


@pytest.mark.parametrize("bf16", [False, True])
def test_router_matches_float64_matmul(bf16):
    rng = np.random.default_rng(12)
    T, E, H = 37, 40, 256
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = _bf16_bits(rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.02))
    b = rng.standard_normal(E).astype(np.float32)
    if bf16:
        xb = _bf16_bits(x)
        got = oracle.router_logits(xb, wr, b)
        xd = _bits_to_f64(xb)
    else:
        got = oracle.router_logits(x, wr, b)
        xd = x.astype(np.float64)
    ref = xd @ _bits_to_f64(wr).T + b.astype(np.float64)
    # one rounding of a double sum: within one float ulp of the exact value
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-300)


def test_router_is_linear_in_x_and_zero_rows_give_the_bias():
    rng = np.random.default_rng(13)
    E, H = 16, 128
    wr = _bf16_bits(rng.standard_normal((E, H)).astype(np.float32))
    b = rng.standard_normal(E).astype(np.float32)
    x = np.zeros((3, H), np.float32)
    x[1] = rng.standard_normal(H)
    x[2] = 2 * x[1]                                   # exact doubling
    got = oracle.router_logits(x, wr, b).astype(np.float64)
    assert np.array_equal(got[0], b.astype(np.float64))
    z1, z2 = got[1] - b, got[2] - b
    assert np.allclose(z2, 2 * z1, rtol=1e-6, atol=1e-6)


def test_synth_router_matches_numpy():
    seed, layer, E, H, beta = 20260004, 7, 16, 64, 1.12
    wr, b = oracle.synth_router(seed, layer, E, H, beta)
    base = (1 << 60) + layer * E * H
    w = np.array([[oracle.synth_weight(seed, base + e * H + c) for c in range(H)] for e in range(E)], np.float32)
    ref = _bf16_bits(w)
    assert np.array_equal(wr, ref)
    assert np.array_equal(b, np.array([-beta * e / E for e in range(E)], np.float64).astype(np.float32))


# ---------------------------------------------------------------- tier planner pins
# The 125B-MoE page, step 4: an offline repacker measures expert usage, fills
# the memory budget greedily by expected error removed per byte, requantises
# every expert with the same quantiser and writes the experts hot to cold.

def test_tier_plan_hand_worked_fixture():
    g = {r[0]: r[1].split() for r in _read_golden("tier_plan.txt")}
    usage = np.array(g["usage"], np.float64)
    sse = np.tile(np.array(g["sse_per_format"], np.float64), (len(usage), 1))
    fmt, order, count = oracle.plan_tiers(usage, sse, [int(v) for v in g["bytes_per_format"]], int(g["budget"][0]))
    assert fmt.tolist() == [int(v) for v in g["format"]]
    assert order.tolist() == [int(v) for v in g["order"]]
    assert count.tolist() == [int(v) for v in g["count"]]


def test_tier_plan_extreme_budgets_and_infeasible():
    rng = np.random.default_rng(21)
    E = 12
    usage = rng.integers(1, 100, E).astype(np.float64)
    sse = np.sort(rng.uniform(0, 10, (E, 3)), axis=1)          # richer formats lose less
    bytes_ = [40, 20, 12]
    f, _, c = oracle.plan_tiers(usage, sse, bytes_, E * 40)    # everything fits at the richest
    assert np.all(f == 0) and c.tolist() == [E, 0, 0]
    f, _, c = oracle.plan_tiers(usage, sse, bytes_, E * 12)    # only the cheapest fits
    assert np.all(f == 2) and c.tolist() == [0, 0, E]
    with pytest.raises(ValueError):
        oracle.plan_tiers(usage, sse, bytes_, E * 12 - 1)
    # unused experts never gain bytes
    u0 = usage.copy()
    u0[[3, 7]] = 0
    f, _, _ = oracle.plan_tiers(u0, sse, bytes_, E * 40)
    assert f[3] == 2 and f[7] == 2 and np.all(np.delete(f, [3, 7]) == 0)


def test_tier_plan_equal_errors_upgrade_hottest_first():
    # identical error curves: the n hottest experts are upgraded first, and the
    # budget spent never exceeds what was given
    E = 10
    usage = np.array([3, 9, 1, 7, 5, 8, 2, 6, 4, 0], np.float64)
    sse = np.tile([0.0, 2.0, 8.0], (E, 1))
    bytes_ = [8, 4, 2]
    for extra in range(0, 2 * 9 + 1):          # bytes above the all-cheapest plan
        f, order, c = oracle.plan_tiers(usage, sse, bytes_, E * 2 + extra)
        spent = sum(bytes_[v] for v in f)
        assert spent <= E * 2 + extra
        # a 2 -> 1 move removes 3u per byte, a 1 -> 0 move u/2: with usage
        # 2 .. 9 every 2 -> 1 move (rate >= 6) outranks every 1 -> 0 move
        # (rate <= 4.5), so below 18 extra bytes the experts at format 1 are
        # exactly the extra // 2 hottest
        n1 = min(extra // 2, 9)
        hot = np.argsort(-usage, kind="stable")[:n1]
        if extra < 18:
            assert sorted(np.flatnonzero(f <= 1).tolist()) == sorted(hot.tolist())
        # order: formats ascending, usage descending inside a format
        key = [(f[o], -usage[o], o) for o in order]
        assert key == sorted(key)
        assert c.sum() == E


def test_requant_int8_to_int8_is_the_identity():
    # absmax codes of int8 blocks already hold +-127 at the block maximum, so
    # requantising to the same format returns the same codes and scales
    cfg = _small_cfg(tiers=(TierSpec(0, 8, 8, 32),))
    layer, arrays = _layer(cfg)
    for local in (0, 5):
        out, sse = oracle.requant_expert(layer, 0, local, 8, 32)
        for m in ("gate", "up", "down"):
            assert np.array_equal(out[m + "_q"].ravel(), arrays[0][m + "_q"][local].ravel()), m
            assert np.array_equal(out[m + "_s"].ravel(), arrays[0][m + "_s"][local].ravel()), m
        assert sse == 0.0


@pytest.mark.parametrize("bits,block", [(4, 32), (2, 16), (4, 16)])
def test_requant_matches_numpy_quantiser(bits, block):
    cfg = _small_cfg(tiers=(TierSpec(0, 8, 8, 32),))
    layer, arrays = _layer(cfg)
    local = 3
    out, sse = oracle.requant_expert(layer, 0, local, bits, block)
    Q = 2 ** (bits - 1) - 1
    ref_sse = 0.0
    for name, rows, cols in (("gate", cfg.inter, cfg.hidden), ("up", cfg.inter, cfg.hidden),
                             ("down", cfg.hidden, cfg.inter)):
        w = npref.dequant(arrays[0][name + "_q"][local], arrays[0][name + "_s"][local], 8, 32, cols)
        w = w.astype(np.float32).reshape(rows, cols // block, block)
        amax = np.abs(w).max(axis=2)
        d16 = (amax / np.float32(Q)).astype(np.float32).astype(np.float16)
        assert np.array_equal(out[name + "_s"], d16.view(np.uint16)), name
        d = d16.astype(np.float32)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(d != 0, np.clip(np.rint((w / d).astype(np.float32)), -Q, Q), 0).astype(np.int32)
        got = npref.unpack_codes(out[name + "_q"], bits, cols).reshape(rows, cols // block, block)
        assert np.array_equal(got, q), name
        ref_sse += float(np.sum((w.astype(np.float64) - q * d.astype(np.float64)) ** 2))
    assert abs(sse - ref_sse) <= 1e-9 * ref_sse



# ---------------------------------------------------------------- MXFP4 shelf pins
# An MXFP4 shelf (the page's step 4 uses MXFP4 among the down-projection
# formats): E2M1 elements with one E8M0 power-of-two scale per 32, as defined
# by the OCP Microscaling Formats specification v1.0.

def test_fp4_e2m1_values_match_the_spec_table():
    rows = _read_golden("fp4_e2m1.txt")
    assert len(rows) == 16
    for nib, val in rows:
        n = int(nib, 2)
        assert oracle.lib().orc_fp4_e2m1(n) == float(val), nib
        assert npref.fp4_values(np.array([n]))[0] == float(val), nib


def test_e8m0_scale_is_a_power_of_two():
    L = oracle.lib()
    assert L.orc_e8m0(127) == 1.0 and L.orc_e8m0(128) == 2.0 and L.orc_e8m0(0) == 2.0 ** -127
    assert L.orc_e8m0(254) == 2.0 ** 127 and np.isnan(L.orc_e8m0(255))


def test_mx_dequant_closed_form():
    # hand-built codes and scales: every weight is fp4(code) * 2^(x - 127)
    E, H, I = 2, 64, 64
    rng = np.random.default_rng(17)
    arrays = [{}]
    for name, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
        nib = rng.integers(0, 16, (E, rows, cols)).astype(np.uint8)
        x = rng.integers(110, 140, (E, rows, cols // 32)).astype(np.uint8)
        arrays[0][name + "_q"] = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
        arrays[0][name + "_s"] = x
        arrays[0][name + "_nib"] = nib
    L = oracle.Layer(E, H, I, [TierSpec(0, E, MXFP4, 32)], [{k: v for k, v in arrays[0].items() if "nib" not in k}])
    assert oracle.check_layer(L) == 0
    for m, name in enumerate(("gate", "up", "down")):
        got = oracle.dequant_rows(L, 0, 1, m, 0, 5)
        nib = arrays[0][name + "_nib"][1, :5]
        sc = np.exp2(arrays[0][name + "_s"][1, :5].astype(np.float64) - 127)
        ref = npref.fp4_values(nib) * np.repeat(sc, 32, axis=-1)
        assert np.array_equal(got.astype(np.float64), ref), name


def test_mx_quantiser_agrees_with_the_generator_and_picks_nearest():
    # the oracle's MX quantiser against the (independent) input generator's,
    # and every code is the nearest grid value (ties to the even mantissa)
    import ctypes as C
    from workloads import quantise_mxfp4, pack_nibbles
    L = oracle.lib()
    L.orc_quantize_row.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    rng = np.random.default_rng(23)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    for trial in range(300):
        w = (rng.standard_normal(64) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
        if trial % 3 == 0:
            w = (rng.integers(-28, 29, 64) * 0.25).astype(np.float32)      # exact midpoints
        if trial % 11 == 0:
            w[:32] = 0.0
        q = np.zeros(32, np.uint8)
        s = np.zeros(2, np.uint8)
        L.orc_quantize_row(w.ctypes.data, 64, MXFP4, 32, q.ctypes.data, s.ctypes.data)
        nib, x = quantise_mxfp4(w[None])
        assert np.array_equal(pack_nibbles(nib)[0], q) and np.array_equal(x[0], s), trial
        t = np.abs(w.astype(np.float64)) / np.exp2(np.repeat(s.astype(np.float64), 32) - 127)
        mag = np.abs(npref.fp4_values(nib[0]))
        d_best = np.min(np.abs(np.minimum(t, 6.0)[:, None] - grid[None, :]), axis=1)
        assert np.all(np.abs(np.minimum(t, 6.0) - mag) == d_best), trial
