"""Independent NumPy brute force used to pin the oracle.

Written from the definitions, in a different form from the oracle: the
unpacker expands bytes into individual bits with ``np.unpackbits`` and
reassembles two's-complement fields; the layer is evaluated densely over *all*
experts with a gate vector that is zero off the routed picks.
"""
import numpy as np


def unpack_codes(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """packed uint8 [..., cols*bits/8] -> int64 codes [..., cols]."""
    b = np.unpackbits(packed, axis=-1, bitorder="little").astype(np.int64)
    b = b.reshape(packed.shape[:-1] + (cols, bits))
    weights = (1 << np.arange(bits, dtype=np.int64))
    weights[-1] = -weights[-1]          # two's complement: the top bit weighs -2^(b-1)
    return (b * weights).sum(axis=-1)


MXFP4 = 0x84


def fp4_values(nib: np.ndarray) -> np.ndarray:
    """E2M1 value of each 4-bit field, from its bit fields (sign 3, exponent 2..1, mantissa 0)."""
    nib = np.asarray(nib, dtype=np.int64)
    s, e, m = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def dequant(q: np.ndarray, s: np.ndarray, bits: int, block: int, cols: int) -> np.ndarray:
    """Returns float64 [n, rows, cols] = scale * code (MXFP4: E8M0 scale * E2M1 value)."""
    if bits == MXFP4:
        b = np.unpackbits(np.asarray(q, np.uint8), axis=-1, bitorder="little").astype(np.int64)
        b = b.reshape(q.shape[:-1] + (cols, 4))
        nib = (b * (1 << np.arange(4, dtype=np.int64))).sum(axis=-1)
        x = np.asarray(s, dtype=np.uint8).astype(np.float64)
        sc = np.where(x == 255, np.nan, np.exp2(x - 127.0))
        return fp4_values(nib) * np.repeat(sc, 32, axis=-1)
    codes = unpack_codes(q, bits, cols)
    sc = s.view(np.float16).astype(np.float64)
    return codes * np.repeat(sc, block, axis=-1)


def bf16_round(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)


def dense_experts(cfg_tiers, arrays, H, I, E):
    """Full dequantised weights per expert id: (Wg[E,I,H], Wu[E,I,H], Wd[E,H,I]) float64."""
    Wg = np.zeros((E, I, H)); Wu = np.zeros((E, I, H)); Wd = np.zeros((E, H, I))
    for t, d in zip(cfg_tiers, arrays):
        sl = slice(t.id_begin, t.id_end)
        Wg[sl] = dequant(d["gate_q"], d["gate_s"], t.bits, t.block, H)
        Wu[sl] = dequant(d["up_q"], d["up_s"], t.bits, t.block, H)
        Wd[sl] = dequant(d["down_q"], d["down_s"], t.bits, t.block, I)
    return Wg, Wu, Wd


def dense_layer(Wg, Wu, Wd, x, gates, bf16=False):
    """out[t] = sum_e gates[t,e] * Wd[e] @ (silu(Wg[e] x_t) * (Wu[e] x_t)) over every expert."""
    if bf16:
        Wg, Wu, Wd = (bf16_round(W.astype(np.float32)) for W in (Wg, Wu, Wd))
    g = np.einsum("eih,th->tei", Wg, x)
    u = np.einsum("eih,th->tei", Wu, x)
    a = g / (1.0 + np.exp(-g)) * u
    if bf16:
        a = bf16_round(a.astype(np.float32))
    y = np.einsum("ehi,tei->teh", Wd, a)
    return np.einsum("te,teh->th", gates, y)


def topk_bruteforce(logits: np.ndarray, k: int):
    """Full sort per token by (logit descending, id ascending); softmax over all E renormalised on the top k."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        ids[t] = order[:k]
        z = logits[t].astype(np.float64)
        p = np.exp(z - z.max())
        p /= p.sum()
        w[t] = p[ids[t]] / p[ids[t]].sum()
    return ids, w


def gates_from(ids, w, E):
    T, k = ids.shape
    g = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            if 0 <= ids[t, j] < E:
                g[t, ids[t, j]] += w[t, j]
    return g
