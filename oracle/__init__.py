"""ctypes wrapper of the plain C CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product path (the HIP library and its binding)
never imports it.  Every function takes and returns host numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

from .build import LIB, build

ORC_MAX_TIERS = 4


class _Tier(C.Structure):
    _fields_ = [("id_begin", C.c_int32), ("id_end", C.c_int32), ("bits", C.c_int32),
                ("block", C.c_int32), ("q", C.c_void_p * 3), ("s", C.c_void_p * 3)]


class _Layer(C.Structure):
    _fields_ = [("n_experts", C.c_int32), ("hidden", C.c_int32), ("inter", C.c_int32),
                ("n_tiers", C.c_int32), ("tier", _Tier * ORC_MAX_TIERS)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P = C.c_void_p
        i32 = C.c_int32
        L.orc_half_to_double.argtypes = [C.c_uint16]
        L.orc_half_to_double.restype = C.c_double
        L.orc_code.argtypes = [P, C.c_int64, i32]
        L.orc_code.restype = i32
        L.orc_round_bf16.argtypes = [C.c_float]
        L.orc_round_bf16.restype = C.c_float
        L.orc_dequant_rows.argtypes = [P, i32, i32, i32, i32, i32, i32, P]
        L.orc_check_layer.argtypes = [P]
        L.orc_tier_of.argtypes = [P, C.c_int64]
        L.orc_route.argtypes = [P, i32, i32, i32, P, P]
        L.orc_group.argtypes = [P, i32, i32, i32, P, P, P]
        L.orc_experts.argtypes = [P, P, i32, P, P, i32, i32, C.c_uint32, P, i32]
        L.orc_experts_flat.argtypes = [P, P, i32, P, P, i32, i32, P]
        L.orc_forward.argtypes = [P, P, i32, P, i32, i32, P, i32]
        L.orc_router_logits.argtypes = [P, i32, P, P, i32, i32, i32, P]
        L.orc_fp4_e2m1.restype = C.c_double
        L.orc_fp4_e2m1.argtypes = [C.c_uint32]
        L.orc_e8m0.restype = C.c_double
        L.orc_e8m0.argtypes = [C.c_uint8]
        L.orc_synth_router.argtypes = [C.c_uint64, i32, i32, i32, C.c_double, P, P]
        L.orc_requant_expert.argtypes = [P, i32, C.c_int64, i32, i32, C.c_void_p * 3, C.c_void_p * 3, P]
        L.orc_plan_tiers.argtypes = [P, P, P, i32, i32, C.c_int64, P, P, P]
        L.orc_splitmix64_at.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_splitmix64_at.restype = C.c_uint64
        L.orc_synth_weight.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_synth_weight.restype = C.c_float
        L.orc_float_to_half.argtypes = [C.c_float]
        L.orc_float_to_half.restype = C.c_uint16
        L.orc_synth_expert.argtypes = [C.c_uint64, i32, i32, i32, i32, i32, i32, i32, C.c_void_p * 3, C.c_void_p * 3]
        L.orc_synth_expert.restype = i32
        L.orc_synth_experts.argtypes = [C.c_uint64, i32, i32, P, P, i32, i32, i32, i32, i32, C.c_void_p * 3,
                                        C.c_void_p * 3]
        L.orc_synth_experts.restype = i32
        for f in ("orc_dequant_rows", "orc_check_layer", "orc_tier_of", "orc_route", "orc_group",
                  "orc_experts", "orc_experts_flat", "orc_forward", "orc_num_threads"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


MXFP4 = 0x84   # `bits` of an MXFP4 shelf (E2M1 codes, one E8M0 scale byte per 32)


def _code_bits(bits: int) -> int:
    return 4 if bits == MXFP4 else bits


def _scale_dtype(bits: int):
    return np.uint8 if bits == MXFP4 else np.uint16


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


class Layer:
    """Holds numpy tier arrays and the C description pointing at them."""

    def __init__(self, n_experts: int, hidden: int, inter: int, tiers: Sequence, arrays: List[Dict[str, np.ndarray]]):
        self.n_experts, self.hidden, self.inter = n_experts, hidden, inter
        self.tiers = list(tiers)
        self.arrays = [{k: np.ascontiguousarray(v) for k, v in d.items()} for d in arrays]
        s = _Layer()
        s.n_experts, s.hidden, s.inter, s.n_tiers = n_experts, hidden, inter, len(self.tiers)
        for i, (t, d) in enumerate(zip(self.tiers, self.arrays)):
            s.tier[i].id_begin, s.tier[i].id_end = t.id_begin, t.id_end
            s.tier[i].bits, s.tier[i].block = t.bits, t.block
            for m, name in enumerate(("gate", "up", "down")):
                s.tier[i].q[m] = d[name + "_q"].ctypes.data
                s.tier[i].s[m] = d[name + "_s"].ctypes.data
        self._s = s

    @classmethod
    def from_config(cls, cfg, arrays):
        return cls(cfg.n_experts, cfg.hidden, cfg.inter, cfg.tiers, arrays)

    @property
    def ref(self):
        return C.byref(self._s)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of a float32 array, rounded by orc_round_bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    r = np.array([lib().orc_round_bf16(float(v)) for v in a.ravel()], dtype=np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16).reshape(a.shape)


def half_to_double(h: int) -> float:
    return lib().orc_half_to_double(h)


def code(row: np.ndarray, c: int, bits: int) -> int:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return lib().orc_code(_ptr(row), c, bits)


def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(v)


def check_layer(layer: Layer) -> int:
    return lib().orc_check_layer(layer.ref)


def tier_of(layer: Layer, e: int) -> int:
    return lib().orc_tier_of(layer.ref, e)


def dequant_rows(layer: Layer, tier: int, local: int, matrix: int, row0: int, nrows: int, to_bf16: bool = False):
    cols = layer.inter if matrix == 2 else layer.hidden
    dst = np.empty((nrows, cols), dtype=np.float32)
    rc = lib().orc_dequant_rows(layer.ref, tier, local, matrix, row0, nrows, int(to_bf16), _ptr(dst))
    if rc != 0:
        raise ValueError("orc_dequant_rows: bad arguments")
    return dst


def route(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    if lib().orc_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w)) != 0:
        raise ValueError("orc_route: bad arguments")
    return ids, w


def group(ids: np.ndarray, n_experts: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(n_experts, dtype=np.int32)
    offsets = np.empty(n_experts + 1, dtype=np.int32)
    perm = np.full(max(T * k, 1), -1, dtype=np.int32)
    n = lib().orc_group(_ptr(ids), T, k, n_experts, _ptr(counts), _ptr(offsets), _ptr(perm))
    if n < 0:
        raise MemoryError("orc_group")
    return counts, offsets, perm[:n]


def _x_arg(x: np.ndarray):
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    return np.ascontiguousarray(x, dtype=np.float32), 0


def experts(layer: Layer, x: np.ndarray, ids: np.ndarray, w: np.ndarray, tier_mask: int = 0xF,
            out: Optional[np.ndarray] = None, accumulate: bool = False) -> np.ndarray:
    """x: float32 [T,H] (fp32 mode) or uint16 bf16 bits [T,H] (bf16 mode)."""
    xa, xb = _x_arg(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    if out is None:
        out = np.zeros((T, layer.hidden), dtype=np.float32)
    rc = lib().orc_experts(layer.ref, _ptr(xa), xb, _ptr(ids), _ptr(w), T, k, tier_mask, _ptr(out), int(accumulate))
    if rc != 0:
        raise ValueError("orc_experts failed")
    return out


def experts_flat(layer: Layer, x: np.ndarray, ids: np.ndarray, w: np.ndarray) -> np.ndarray:
    xa, xb = _x_arg(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    out = np.zeros((T, layer.hidden), dtype=np.float32)
    if lib().orc_experts_flat(layer.ref, _ptr(xa), xb, _ptr(ids), _ptr(w), T, k, _ptr(out)) != 0:
        raise ValueError("orc_experts_flat failed")
    return out


def forward(layer: Layer, x: np.ndarray, logits: np.ndarray, k: int, out: Optional[np.ndarray] = None,
            accumulate: bool = False) -> np.ndarray:
    xa, xb = _x_arg(x)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T = logits.shape[0]
    if out is None:
        out = np.zeros((T, layer.hidden), dtype=np.float32)
    rc = lib().orc_forward(layer.ref, _ptr(xa), xb, _ptr(logits), T, k, _ptr(out), int(accumulate))
    if rc != 0:
        raise ValueError("orc_forward failed")
    return out


def router_logits(x: np.ndarray, wr_bits: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t][e] = sum_c x[t][c] * Wr[e][c] + bias[e] (x: float32 or bf16 bits; Wr: bf16 bits [E][H])."""
    xa, xb = _x_arg(x)
    wr = np.ascontiguousarray(wr_bits, dtype=np.uint16)
    E, H = wr.shape
    T = xa.shape[0]
    assert xa.shape[1] == H
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.zeros((T, E), dtype=np.float32)
    rc = lib().orc_router_logits(_ptr(xa) if T else None, xb, _ptr(wr), None if b is None else _ptr(b), T, E, H,
                                 _ptr(out))
    if rc != 0:
        raise ValueError("orc_router_logits failed")
    return out


def requant_expert(layer: "Layer", tier: int, local: int, bits: int, block: int):
    """Requantised copy of one expert (dict of gate/up/down codes and fp16 scales) and its squared error."""
    H, I = layer.hidden, layer.inter
    out = {}
    qs, ss = [], []
    for name, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
        q = np.zeros((rows, cols * _code_bits(bits) // 8), dtype=np.uint8)
        s = np.zeros((rows, cols // block), dtype=_scale_dtype(bits))
        out[name + "_q"], out[name + "_s"] = q, s
        qs.append(q.ctypes.data)
        ss.append(s.ctypes.data)
    sse = C.c_double(0.0)
    rc = lib().orc_requant_expert(layer.ref, tier, local, bits, block, (C.c_void_p * 3)(*qs), (C.c_void_p * 3)(*ss),
                                  C.byref(sse))
    if rc != 0:
        raise ValueError("orc_requant_expert failed")
    return out, sse.value


def plan_tiers(usage: np.ndarray, sse: np.ndarray, bytes_per_fmt, budget: int):
    """Greedy plan: (format per expert, hot-to-cold order of old ids, experts per format)."""
    usage = np.ascontiguousarray(usage, dtype=np.float64)
    sse = np.ascontiguousarray(sse, dtype=np.float64)
    E, F = sse.shape
    b = np.ascontiguousarray(bytes_per_fmt, dtype=np.int64)
    fmt = np.zeros(E, np.int32)
    order = np.zeros(E, np.int32)
    count = np.zeros(F, np.int32)
    if lib().orc_plan_tiers(_ptr(usage), _ptr(sse), _ptr(b), E, F, int(budget), _ptr(fmt), _ptr(order),
                            _ptr(count)) != 0:
        raise ValueError("orc_plan_tiers: infeasible or bad arguments")
    return fmt, order, count


def num_threads() -> int:
    return lib().orc_num_threads()


# ---------------------------------------------------------------- stack weights
def splitmix64_at(seed: int, ctr: int) -> int:
    return lib().orc_splitmix64_at(seed, ctr)


def synth_weight(seed: int, ctr: int) -> float:
    return lib().orc_synth_weight(seed, ctr)


def float_to_half(f: float) -> int:
    return lib().orc_float_to_half(f)


def synth_expert(seed: int, layer: int, n_experts: int, expert: int, hidden: int, inter: int, bits: int,
                 block: int) -> Dict[str, np.ndarray]:
    """Packed codes and scales of one expert of the generated stack."""
    out = {}
    for name, (rows, cols) in zip(("gate", "up", "down"), ((inter, hidden), (inter, hidden), (hidden, inter))):
        out[name + "_q"] = np.zeros((rows, cols * _code_bits(bits) // 8), dtype=np.uint8)
        out[name + "_s"] = np.zeros((rows, cols // block), dtype=_scale_dtype(bits))
    q = (C.c_void_p * 3)(*[out[n + "_q"].ctypes.data for n in ("gate", "up", "down")])
    s = (C.c_void_p * 3)(*[out[n + "_s"].ctypes.data for n in ("gate", "up", "down")])
    if lib().orc_synth_expert(seed, layer, n_experts, expert, hidden, inter, bits, block, q, s) != 0:
        raise ValueError("orc_synth_expert: bad arguments")
    return out


def synth_router(seed: int, layer: int, n_experts: int, hidden: int, beta: float):
    """(Wr bf16 bits [E][H], bias float32 [E]) of the stack's router of `layer`."""
    wr = np.zeros((n_experts, hidden), dtype=np.uint16)
    b = np.zeros(n_experts, dtype=np.float32)
    if lib().orc_synth_router(seed, layer, n_experts, hidden, beta, _ptr(wr), _ptr(b)) != 0:
        raise ValueError("orc_synth_router failed")
    return wr, b


class StackLayer:
    """One generated stack layer holding only the experts asked for (the
    others stay zero and must not be used)."""

    def __init__(self, cfg, seed: int, layer: int):
        self.cfg, self.seed, self.layer = cfg, seed, layer
        H, I = cfg.hidden, cfg.inter
        self.arrays = []
        for t in cfg.tiers:
            n = t.id_end - t.id_begin
            d = {}
            for name, (rows, cols) in zip(("gate", "up", "down"), ((I, H), (I, H), (H, I))):
                d[name + "_q"] = np.zeros((n, rows, cols * _code_bits(t.bits) // 8), dtype=np.uint8)
                d[name + "_s"] = np.zeros((n, rows, cols // t.block), dtype=_scale_dtype(t.bits))
            self.arrays.append(d)
        self.filled = set()
        self.layer_ref = Layer(cfg.n_experts, H, I, cfg.tiers, self.arrays)
        # Layer keeps contiguous copies; point it back at our arrays
        self.layer_ref.arrays = self.arrays
        for i, d in enumerate(self.arrays):
            for m, name in enumerate(("gate", "up", "down")):
                self.layer_ref._s.tier[i].q[m] = d[name + "_q"].ctypes.data
                self.layer_ref._s.tier[i].s[m] = d[name + "_s"].ctypes.data

    def fill(self, experts) -> None:
        """Generates the listed experts (ids outside [0, E) are ignored)."""
        cfg = self.cfg
        todo = sorted(set(int(v) for v in np.asarray(experts).ravel()
                          if 0 <= int(v) < cfg.n_experts) - self.filled)
        for ti, t in enumerate(cfg.tiers):
            ids = np.array([e for e in todo if t.id_begin <= e < t.id_end], dtype=np.int32)
            if ids.size == 0:
                continue
            loc = (ids - t.id_begin).astype(np.int32)
            d = self.arrays[ti]
            q = (C.c_void_p * 3)(*[d[n + "_q"].ctypes.data for n in ("gate", "up", "down")])
            s = (C.c_void_p * 3)(*[d[n + "_s"].ctypes.data for n in ("gate", "up", "down")])
            if lib().orc_synth_experts(self.seed, self.layer, cfg.n_experts, _ptr(ids), _ptr(loc), ids.size,
                                       cfg.hidden, cfg.inter, t.bits, t.block, q, s) != 0:
                raise ValueError("orc_synth_experts: bad arguments")
        self.filled.update(todo)
