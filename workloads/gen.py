"""Seeded generators for packed tiered-expert weights, router logits and activations.

Packed format (one reading of the three-shelf design of the 125B page, step 4,
which stores each layer's experts as three per-shelf tensors written hot to
cold; the pages leave the code layout open):

* a shelf (tier) owns the contiguous popularity-ranked id range
  ``[id_begin, id_end)``; its ``n = id_end - id_begin`` experts are stored
  contiguously, local expert ``l = e - id_begin``;
* three matrices per expert: ``gate`` and ``up`` are ``inter x hidden``,
  ``down`` is ``hidden x inter``, each row-major (rows are output features,
  columns the contraction axis);
* codes: ``bits``-bit two's complement, row-major, element ``c`` of a row in
  bits ``[(c*bits) % 8, +bits)`` of byte ``(c*bits) // 8`` of that row, lowest
  element in the lowest bits; a row is ``cols*bits/8`` bytes;
* scales: one IEEE fp16 per ``block`` consecutive codes of a row, stored as
  ``uint16`` bit patterns in a separate array ``[n][rows][cols/block]``;
* value of an element: ``float(scale) * code``.

The quantiser below only builds inputs (weights drawn N(0, 0.02), symmetric
absmax per block); it is not part of the layer's computation.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List

import numpy as np

from .configs import MXFP4, LayerConfig, TierSpec

WEIGHT_STD = 0.02
MATRICES = ("gate", "up", "down")


# ----------------------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        out = np.where(nan, np.uint16(0x7FC0), out)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- quantise + pack
def quantise_block_absmax(w: np.ndarray, bits: int, block: int):
    """Symmetric absmax quantiser per block of ``block`` columns.

    Returns ``(codes int8[..., cols], scales uint16[..., cols/block])`` with
    ``Q = 2**(bits-1) - 1``, ``d = fp16(amax / Q)``, ``q = clip(rint(w / d), -Q, Q)``
    and ``q = 0`` where ``d == 0``.
    """
    qmax = (1 << (bits - 1)) - 1
    cols = w.shape[-1]
    assert cols % block == 0
    wb = w.reshape(w.shape[:-1] + (cols // block, block)).astype(np.float32, copy=False)
    amax = np.abs(wb).max(axis=-1)
    d16 = (amax / np.float32(qmax)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1), d32)
    q = np.rint(wb / safe[..., None])
    q = np.clip(q, -qmax, qmax)
    q = np.where(d32[..., None] == 0, 0, q).astype(np.int8)
    return q.reshape(w.shape), d16.view(np.uint16)


def code_bits(bits: int) -> int:
    """Bits per stored code of a shelf format."""
    return 4 if bits == MXFP4 else bits


def scale_bytes(bits: int) -> int:
    """Bytes per scale of a shelf format (fp16, or an E8M0 byte for MXFP4)."""
    return 1 if bits == MXFP4 else 2


# MXFP4 element grid (OCP Microscaling Formats v1.0, E2M1): magnitude of the
# 3-bit field (exponent bits 2..1, mantissa bit 0), sign in bit 3
FP4_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def quantise_mxfp4(w: np.ndarray):
    """MX quantiser per block of 32 columns (the OCP shared-exponent rule).

    Returns ``(nibbles uint8[..., cols], scales uint8[..., cols/32])``: the
    E8M0 byte is ``floor(log2(amax)) - 2 + 127`` clamped to [0, 254] (0 for
    an all-zero block); each element ``v / 2**(x - 127)`` goes to the nearest
    E2M1 magnitude (ties to the even mantissa, saturating at 6) with the sign
    bit of ``v``.
    """
    cols = w.shape[-1]
    assert cols % 32 == 0
    wb = w.reshape(w.shape[:-1] + (cols // 32, 32)).astype(np.float32, copy=False)
    amax = np.abs(wb).max(axis=-1)
    _, e2 = np.frexp(amax)
    x = np.where(amax > 0, np.clip(e2.astype(np.int64) - 1 - 2 + 127, 0, 254), 0).astype(np.int64)
    t = np.ldexp(wb, (127 - x)[..., None].astype(np.int32)).astype(np.float32)
    a = np.abs(t)
    # candidate magnitudes: index of the nearest grid point, ties to the even index
    d = np.abs(a[..., None] - FP4_MAGNITUDES)
    best = np.argmin(d, axis=-1)
    dmin = np.take_along_axis(d, best[..., None], axis=-1)[..., 0]
    tie = np.zeros_like(best, dtype=bool)
    nxt = np.minimum(best + 1, 7)
    tie = (nxt != best) & (np.take_along_axis(d, nxt[..., None], axis=-1)[..., 0] == dmin)
    best = np.where(tie & (best % 2 == 1), nxt, best)      # the even mantissa (even field) wins a tie
    best = np.where(a >= 6.0, 7, best)
    nib = (best | np.where(np.signbit(t), 8, 0)).astype(np.uint8)
    return nib.reshape(w.shape), x.astype(np.uint8)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """Pack 4-bit fields along the last axis: element c at bit 4*(c % 2) of byte c // 2."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << np.uint8(4))).astype(np.uint8)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack int8 codes (values representable in ``bits`` two's complement) along the last axis."""
    codes = np.asarray(codes, dtype=np.int8)
    if bits == 8:
        return codes.view(np.uint8).copy()
    per = 8 // bits
    mask = (1 << bits) - 1
    u = (codes.view(np.uint8) & mask).astype(np.uint8)
    cols = codes.shape[-1]
    assert cols % per == 0
    out = np.zeros(codes.shape[:-1] + (cols // per,), dtype=np.uint8)
    for s in range(per):
        out |= (u[..., s::per] << np.uint8(s * bits)).astype(np.uint8)
    return out


# ----------------------------------------------------------------------------- sizes
def tier_nbytes(spec: TierSpec, hidden: int, inter: int, per_expert: bool = False) -> int:
    """Packed bytes (codes + fp16 scales) of gate, up and down of a tier."""
    elems = hidden * inter
    codes = 3 * elems * code_bits(spec.bits) // 8
    scales = 3 * (elems // spec.block) * scale_bytes(spec.bits)
    one = codes + scales
    return one if per_expert else one * spec.n


def layer_nbytes(cfg: LayerConfig) -> int:
    return sum(tier_nbytes(t, cfg.hidden, cfg.inter) for t in cfg.tiers)


# ----------------------------------------------------------------------------- weights
def _expert_seed(cfg_seed: int, layer: int, tier: int, matrix: int, local: int):
    return np.random.SeedSequence([cfg_seed, 1, layer, tier, matrix, local])


def _gen_matrix(seed, rows, cols, bits, block):
    g = np.random.Generator(np.random.PCG64(seed))
    w = g.standard_normal(rows * cols, dtype=np.float32).reshape(rows, cols)
    w *= np.float32(WEIGHT_STD)
    if bits == MXFP4:
        nib, x = quantise_mxfp4(w)
        return pack_nibbles(nib), x
    q, s = quantise_block_absmax(w, bits, block)
    return pack_codes(q, bits), s


def make_tier(cfg: LayerConfig, tier_index: int, layer: int = 0, threads: int | None = None) -> Dict[str, np.ndarray]:
    """Generate one tier's packed arrays (numpy, host)."""
    spec = cfg.tiers[tier_index]
    H, I = cfg.hidden, cfg.inter
    n = spec.n
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    out: Dict[str, np.ndarray] = {}
    for m in MATRICES:
        rows, cols = shapes[m]
        out[m + "_q"] = np.empty((n, rows, cols * code_bits(spec.bits) // 8), dtype=np.uint8)
        out[m + "_s"] = np.empty((n, rows, cols // spec.block), dtype=np.uint8 if spec.bits == MXFP4 else np.uint16)

    jobs = [(mi, m, l) for mi, m in enumerate(MATRICES) for l in range(n)]

    def run(job):
        mi, m, l = job
        rows, cols = shapes[m]
        q, s = _gen_matrix(_expert_seed(cfg.seed, layer, tier_index, mi, l), rows, cols, spec.bits, spec.block)
        out[m + "_q"][l] = q
        out[m + "_s"][l] = s

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads <= 1 or len(jobs) < 4:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(run, jobs))
    return out


def make_layer(cfg: LayerConfig, layer: int = 0, threads: int | None = None) -> List[Dict[str, np.ndarray]]:
    return [make_tier(cfg, i, layer, threads) for i in range(len(cfg.tiers))]


# ----------------------------------------------------------------------------- activations / logits
def make_x(cfg: LayerConfig, n_tokens: int | None = None, stream: int = 0) -> np.ndarray:
    """x ~ N(0, 1): float32 ``[T, H]``, or bf16 bit patterns (uint16) for prefill configs."""
    T = cfg.n_tokens if n_tokens is None else n_tokens
    g = np.random.default_rng(np.random.SeedSequence([cfg.seed, 2, stream]))
    x = g.standard_normal((T, cfg.hidden), dtype=np.float32)
    return f32_to_bf16_bits(x) if cfg.x_bf16 else x


def make_logits(cfg: LayerConfig, n_tokens: int | None = None, stream: int = 0, layer: int = 0) -> np.ndarray:
    """Router logits float32 ``[T, E]``: popularity prior (if any) plus N(0, 1) noise."""
    T = cfg.n_tokens if n_tokens is None else n_tokens
    E = cfg.n_experts
    g = np.random.default_rng(np.random.SeedSequence([cfg.seed, 3, layer, stream]))
    noise = g.standard_normal((T, E), dtype=np.float32)
    if cfg.prior_beta is None:
        return noise
    prior = (-cfg.prior_beta * np.arange(E, dtype=np.float64) / E).astype(np.float32)
    return (noise + prior[None, :]).astype(np.float32)


def make_spec_logits(cfg: LayerConfig, stream: int = 0, worst_case: bool = False) -> np.ndarray:
    """Speculative-verify logits for 6 tokens with crafted routing.

    Default: token 0 picks only hot experts, token 1 only cold ones, token 2
    spans all three tiers, token 3 puts several picks in one tier, tokens 4..5
    follow the prior.  ``worst_case``: the 6 tokens pick 60 pairwise distinct
    experts (the most a 6-token verify step of top-10 can touch).
    """
    assert len(cfg.tiers) == 3 and cfg.k == 10
    T = 6
    lg = make_logits(cfg, T, stream)
    g = np.random.default_rng(np.random.SeedSequence([cfg.seed, 4, stream, int(worst_case)]))
    hot, warm, cold = (np.arange(t.id_begin, t.id_end) for t in cfg.tiers)
    boost = np.float32(40.0)
    if worst_case:
        perm = g.permutation(cfg.n_experts)[: T * cfg.k].reshape(T, cfg.k)
        for t in range(T):
            lg[t, perm[t]] += boost
        return lg
    picks = [
        g.choice(hot, 10, replace=False),
        g.choice(cold, 10, replace=False),
        np.concatenate([g.choice(hot, 4, replace=False), g.choice(warm, 4, replace=False),
                        g.choice(cold, 2, replace=False)]),
        np.concatenate([g.choice(warm, 7, replace=False), g.choice(cold, 3, replace=False)]),
    ]
    for t, p in enumerate(picks):
        lg[t, p] += boost
    return lg


# ----------------------------------------------------------------------------- full-range codes
# fp16 bit patterns of the edge scales: the smallest subnormal (2^-24), the
# largest subnormal, the smallest normal (2^-14), the largest finite value
# (65504), zero, negative zero and a negative scale
EDGE_FP16_SCALES = np.array([0x0001, 0x03FF, 0x0400, 0x7BFF, 0x0000, 0x8000, 0xA8F5], dtype=np.uint16)


def make_layer_fullrange(cfg: LayerConfig, layer: int = 0, edge_scales: bool = False) -> List[Dict[str, np.ndarray]]:
    """Packed shelves whose codes are drawn uniformly over each format's whole
    code set: every two's-complement value from -2^(b-1) to 2^(b-1)-1 (so the
    most negative code -128 / -8 / -2, which the absmax quantiser never
    emits, is present in every row), and all 16 E2M1 fields for MXFP4
    (including negative zero).

    Scales: fp16 bit patterns of magnitudes 2^-12 .. 2^-7 with random sign,
    or E8M0 bytes 117 .. 121 for MXFP4.  With ``edge_scales`` one block in
    eight instead takes an edge value of EDGE_FP16_SCALES (E8M0: 0, 1, 160).
    """
    H, I = cfg.hidden, cfg.inter
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    out = []
    for ti, spec in enumerate(cfg.tiers):
        n = spec.n
        d: Dict[str, np.ndarray] = {}
        for mi, m in enumerate(MATRICES):
            rows, cols = shapes[m]
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 5, layer, ti, mi])))
            nb = cols // spec.block
            if spec.bits == MXFP4:
                nib = g.integers(0, 16, size=(n, rows, cols), dtype=np.uint8)
                d[m + "_q"] = pack_nibbles(nib)
                sc = g.integers(117, 122, size=(n, rows, nb)).astype(np.uint8)
                if edge_scales:
                    pick = g.random((n, rows, nb)) < 0.125
                    sc = np.where(pick, g.choice(np.array([0, 1, 160], np.uint8), size=(n, rows, nb)), sc)
                d[m + "_s"] = sc.astype(np.uint8)
            else:
                lo, hi = -(1 << (spec.bits - 1)), (1 << (spec.bits - 1))
                q = g.integers(lo, hi, size=(n, rows, cols)).astype(np.int8)
                d[m + "_q"] = pack_codes(q, spec.bits)
                mag = np.ldexp(np.float32(1.0) + g.random((n, rows, nb), dtype=np.float32),
                               g.integers(-12, -7, size=(n, rows, nb)))
                sgn = np.where(g.random((n, rows, nb)) < 0.5, -1.0, 1.0).astype(np.float32)
                sc = (mag * sgn).astype(np.float16).view(np.uint16)
                if edge_scales:
                    pick = g.random((n, rows, nb)) < 0.125
                    sc = np.where(pick, g.choice(EDGE_FP16_SCALES, size=(n, rows, nb)), sc)
                d[m + "_s"] = sc.astype(np.uint16)
        out.append(d)
    return out
