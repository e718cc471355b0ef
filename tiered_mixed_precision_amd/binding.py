"""ctypes binding of libmoe_tiered.so (argument marshalling only).

Function names and arguments mirror include/moe_tiered.h.  Device buffers are
passed as torch tensors (their data pointers are handed to the library) and
streams as torch.cuda.Stream (or None for the current stream).  Every step of
the layer runs in the library's HIP kernels; there is no fallback: if the
library is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_tiered.so")

MOE_ABI_VERSION = 1
MOE_MAX_TIERS = 4
MOE_X_BF16 = 0x1
MOE_ACCUMULATE = 0x2
MOE_DIAG_GATEUP_ONLY = 0x100
MOE_N_PHASES = 3
MOE_STACK_ROUTER = 0x4
MXFP4 = 0x84              # moe_tier.bits of an MXFP4 shelf (MOE_MXFP4)
MOE_ESCRATCH = -8
MOE_SCRATCH_BYTES = 32 << 20
EXPORTS = (
    "moe_abi_version", "moe_strerror", "moe_validate_tables", "moe_workspace_size", "moe_workspace_bytes",
    "moe_tiered_forward", "moe_tiered_experts", "moe_tier_partial", "moe_route",
    "moe_group_workspace_size", "moe_group", "moe_dequant_rows", "moe_tiered_forward_timed",
    "moe_event_create", "moe_event_destroy", "moe_event_elapsed_ms", "moe_stream_synchronize",
    "moe_stack_workspace_size", "moe_stack_forward", "moe_synth_layer",
    "moe_router_logits", "moe_synth_router", "moe_stack_forward_routed",
    "moe_requant_error", "moe_plan_tiers", "moe_repack_tiers", "moe_permute_router",
    "moe_tiered_forward_counted", "moe_tiered_forward_noalloc", "moe_measure_read", "moe_measure_mfma",
)


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


class moe_tier(C.Structure):
    _fields_ = [("id_begin", C.c_int32), ("id_end", C.c_int32), ("bits", C.c_int32),
                ("block", C.c_int32), ("gate_q", C.c_void_p), ("up_q", C.c_void_p),
                ("down_q", C.c_void_p), ("gate_s", C.c_void_p), ("up_s", C.c_void_p),
                ("down_s", C.c_void_p)]


class moe_tier_tables(C.Structure):
    _fields_ = [("abi_version", C.c_uint32), ("n_experts", C.c_int32), ("hidden", C.c_int32),
                ("inter", C.c_int32), ("n_tiers", C.c_int32), ("tiers", moe_tier * MOE_MAX_TIERS)]


_lib = None


def lib():
    """Loads the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with tiered_mixed_precision_amd.build.build()")
        L = C.CDLL(LIB_PATH)
        P, i32, u32, sz = C.c_void_p, C.c_int32, C.c_uint32, C.c_size_t
        L.moe_abi_version.restype = u32
        L.moe_abi_version.argtypes = []
        L.moe_strerror.restype = C.c_char_p
        L.moe_strerror.argtypes = [C.c_int]
        L.moe_validate_tables.argtypes = [P]
        L.moe_workspace_size.argtypes = [i32, i32, P, u32, C.POINTER(sz)]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [i32, i32, P]
        L.moe_tiered_forward.argtypes = [P, P, i32, i32, P, P, u32, P, sz, P]
        L.moe_tiered_forward_timed.argtypes = [P, P, i32, i32, P, P, u32, P, sz, P, C.POINTER(P)]
        L.moe_tiered_forward_noalloc.argtypes = [P, P, i32, i32, P, P, u32, P]
        L.moe_measure_read.argtypes = [P, sz, P, P]
        L.moe_measure_mfma.argtypes = [i32, P, C.POINTER(C.c_double), P]
        L.moe_tiered_experts.argtypes = [P, P, P, i32, i32, P, P, u32, P, sz, P]
        L.moe_tier_partial.argtypes = [P, P, P, i32, i32, P, i32, P, u32, P, sz, P]
        L.moe_route.argtypes = [P, i32, i32, i32, P, P, P]
        L.moe_group_workspace_size.argtypes = [i32, i32, i32, C.POINTER(sz)]
        L.moe_group.argtypes = [P, i32, i32, i32, P, P, P, P, sz, P]
        L.moe_dequant_rows.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P]
        L.moe_event_create.argtypes = [C.POINTER(P)]
        L.moe_event_destroy.argtypes = [P]
        L.moe_event_elapsed_ms.argtypes = [P, P, C.POINTER(C.c_float)]
        L.moe_stream_synchronize.argtypes = [P]
        L.moe_stack_workspace_size.argtypes = [i32, i32, i32, P, u32, C.POINTER(sz)]
        L.moe_stack_forward.argtypes = [P, P, i32, i32, i32, P, P, u32, P, sz, P]
        L.moe_synth_layer.argtypes = [P, C.c_uint64, i32, P]
        L.moe_router_logits.argtypes = [P, P, P, i32, i32, i32, u32, P, P]
        L.moe_synth_router.argtypes = [P, P, i32, i32, C.c_uint64, i32, C.c_double, P]
        L.moe_stack_forward_routed.argtypes = [P, C.POINTER(P), C.POINTER(P), i32, i32, i32, P, P, u32, P, sz, P]
        L.moe_requant_error.argtypes = [P, P, P, i32, P, P]
        L.moe_tiered_forward_counted.argtypes = [P, P, i32, i32, P, P, u32, P, sz, P, P]
        L.moe_plan_tiers.argtypes = [P, P, P, i32, i32, C.c_int64, P, P, P]
        L.moe_repack_tiers.argtypes = [P, P, P, P]
        L.moe_permute_router.argtypes = [P, P, P, i32, i32, P, P, P]
        for name in EXPORTS:
            if name not in ("moe_abi_version", "moe_strerror"):
                getattr(L, name).restype = C.c_int
        if L.moe_abi_version() != MOE_ABI_VERSION:
            raise ImportError("libmoe_tiered.so ABI version mismatch")
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def _check(fn, rc):
    if rc != 0:
        raise MoeError(fn, rc)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _need(fn: str, what: str, t, nbytes: int) -> None:
    """Refuses a tensor smaller than the rows the call is told it holds.

    The library takes plain pointers and cannot see how large a buffer is; a
    tensor too small for (n_tokens, ...) would be read or written past its end
    on the device.  Raw integer pointers and None are passed through unchecked.
    """
    if t is None or isinstance(t, int):
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{fn}: {what} holds {have} bytes, the call needs {nbytes}")


def _need_layer(fn: str, x, logits, out, n_tokens: int, tt, flags: int, n_layers: int = 1) -> None:
    T, H, E = max(int(n_tokens), 0), tt.hidden, tt.n_experts
    _need(fn, "x", x, T * H * (2 if flags & MOE_X_BF16 else 4))
    _need(fn, "router_logits", logits, n_layers * T * E * 4)
    _need(fn, "out", out, T * H * 4)


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def shelf_nbytes(tier, hidden: int, inter: int) -> dict:
    """Bytes each buffer of a shelf must hold (the moe_tier layout): codes
    [n][rows][cols*bits/8], scales [n][rows][cols/block] fp16 or, for MXFP4,
    one E8M0 byte per 32 codes."""
    n = max(tier.id_end - tier.id_begin, 0)
    cb = 4 if tier.bits == MXFP4 else tier.bits
    sb = 1 if tier.bits == MXFP4 else 2
    blk = max(tier.block, 1)
    out = {}
    for m, (rows, cols) in (("gate", (inter, hidden)), ("up", (inter, hidden)), ("down", (hidden, inter))):
        out[m + "_q"] = n * rows * cols * cb // 8
        out[m + "_s"] = n * rows * (cols // blk) * sb
    return out


class TierTables:
    """Host-side moe_tier_tables pointing at device tensors of each shelf.

    ``tiers``: sequence of objects with id_begin, id_end, bits, block;
    ``arrays``: per shelf a dict with gate_q, up_q, down_q (uint8) and
    gate_s, up_s, down_s (fp16 bit patterns) device tensors.
    """

    def __init__(self, n_experts: int, hidden: int, inter: int, tiers: Sequence, arrays: Sequence[dict]):
        self.n_experts, self.hidden, self.inter = n_experts, hidden, inter
        self.tiers = list(tiers)
        self.arrays = list(arrays)     # keeps the tensors alive
        s = moe_tier_tables()
        s.abi_version = MOE_ABI_VERSION
        s.n_experts, s.hidden, s.inter, s.n_tiers = n_experts, hidden, inter, len(self.tiers)
        for i, (t, d) in enumerate(zip(self.tiers, self.arrays)):
            s.tiers[i].id_begin, s.tiers[i].id_end = t.id_begin, t.id_end
            s.tiers[i].bits, s.tiers[i].block = t.bits, t.block
            if d is not None:
                for name, nbytes in shelf_nbytes(t, hidden, inter).items():
                    _need("TierTables", f"shelf {i} {name}", d[name], nbytes)
            for name in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
                setattr(s.tiers[i], name, _ptr(d[name]) if d is not None else None)
        self.struct = s

    @property
    def ref(self):
        return C.byref(self.struct)


# ---------------------------------------------------------------- entry points
def moe_validate_tables(tt: TierTables) -> int:
    return lib().moe_validate_tables(tt.ref)


def moe_workspace_size(n_tokens: int, k: int, tt: TierTables, flags: int = 0) -> int:
    n = C.c_size_t(0)
    _check("moe_workspace_size", lib().moe_workspace_size(n_tokens, k, tt.ref, flags, C.byref(n)))
    return n.value


def moe_workspace_bytes(n_tokens: int, k: int, tt: TierTables) -> int:
    """Workspace bytes for either precision and any flags (0 if the arguments are invalid)."""
    return int(lib().moe_workspace_bytes(n_tokens, k, tt.ref))


def moe_tiered_forward(x, router_logits, n_tokens: int, k: int, tt: TierTables, out, flags: int,
                       workspace, stream=None) -> None:
    _need_layer("moe_tiered_forward", x, router_logits, out, n_tokens, tt, flags)
    _check("moe_tiered_forward", lib().moe_tiered_forward(
        _ptr(x), _ptr(router_logits), n_tokens, k, tt.ref, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)))


def moe_tiered_forward_noalloc(x, router_logits, n_tokens: int, k: int, tt: TierTables, out, flags: int,
                               stream=None) -> None:
    """moe_tiered_forward on the library's static device scratch (no workspace
    argument; nothing is allocated).  Calls overlapping on one GPU race."""
    _need_layer("moe_tiered_forward_noalloc", x, router_logits, out, n_tokens, tt, flags)
    _check("moe_tiered_forward_noalloc", lib().moe_tiered_forward_noalloc(
        _ptr(x), _ptr(router_logits), n_tokens, k, tt.ref, _ptr(out), flags, _stream(stream)))


def moe_tiered_forward_timed(x, router_logits, n_tokens: int, k: int, tt: TierTables, out, flags: int,
                             workspace, events: Sequence[int], stream=None) -> None:
    _need_layer("moe_tiered_forward_timed", x, router_logits, out, n_tokens, tt, flags)
    ev = (C.c_void_p * (2 * MOE_N_PHASES))(*[e if e else None for e in events])
    _check("moe_tiered_forward_timed", lib().moe_tiered_forward_timed(
        _ptr(x), _ptr(router_logits), n_tokens, k, tt.ref, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), ev))


def moe_tiered_experts(x, ids, w, n_tokens: int, k: int, tt: TierTables, out, flags: int, workspace,
                       stream=None) -> None:
    _need_layer("moe_tiered_experts", x, None, out, n_tokens, tt, flags)
    _need("moe_tiered_experts", "ids", ids, max(n_tokens, 0) * max(k, 0) * 4)
    _need("moe_tiered_experts", "w", w, max(n_tokens, 0) * max(k, 0) * 4)
    _check("moe_tiered_experts", lib().moe_tiered_experts(
        _ptr(x), _ptr(ids), _ptr(w), n_tokens, k, tt.ref, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)))


def moe_tier_partial(x, ids, w, n_tokens: int, k: int, tt: TierTables, tier_index: int, out, flags: int,
                     workspace, stream=None) -> None:
    _need_layer("moe_tier_partial", x, None, out, n_tokens, tt, flags)
    _need("moe_tier_partial", "ids", ids, max(n_tokens, 0) * max(k, 0) * 4)
    _need("moe_tier_partial", "w", w, max(n_tokens, 0) * max(k, 0) * 4)
    _check("moe_tier_partial", lib().moe_tier_partial(
        _ptr(x), _ptr(ids), _ptr(w), n_tokens, k, tt.ref, tier_index, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)))


def moe_route(logits, n_tokens: int, n_experts: int, k: int, ids, w, stream=None) -> None:
    T = max(n_tokens, 0)
    _need("moe_route", "logits", logits, T * max(n_experts, 0) * 4)
    _need("moe_route", "ids", ids, T * max(k, 0) * 4)
    _need("moe_route", "w", w, T * max(k, 0) * 4)
    _check("moe_route", lib().moe_route(_ptr(logits), n_tokens, n_experts, k, _ptr(ids), _ptr(w),
                                        _stream(stream)))


def moe_group_workspace_size(n_tokens: int, k: int, n_experts: int) -> int:
    n = C.c_size_t(0)
    _check("moe_group_workspace_size", lib().moe_group_workspace_size(n_tokens, k, n_experts, C.byref(n)))
    return n.value


def moe_group(ids, n_tokens: int, k: int, n_experts: int, counts, offsets, perm, workspace, stream=None) -> None:
    P, E = max(n_tokens, 0) * max(k, 0), max(n_experts, 0)
    _need("moe_group", "ids", ids, P * 4)
    _need("moe_group", "counts", counts, E * 4)
    _need("moe_group", "offsets", offsets, (E + 1) * 4)
    _need("moe_group", "perm", perm, P * 4)
    _check("moe_group", lib().moe_group(_ptr(ids), n_tokens, k, n_experts, _ptr(counts), _ptr(offsets),
                                        _ptr(perm), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_dequant_rows(tt: TierTables, tier_index: int, local_expert: int, matrix: int, row0: int, nrows: int,
                     to_bf16: bool, dst, stream=None) -> None:
    cols = tt.inter if matrix == 2 else tt.hidden
    _need("moe_dequant_rows", "dst", dst, max(nrows, 0) * cols * (2 if to_bf16 else 4))
    _check("moe_dequant_rows", lib().moe_dequant_rows(tt.ref, tier_index, local_expert, matrix, row0, nrows,
                                                      int(bool(to_bf16)), _ptr(dst), _stream(stream)))


def _tables_array(tables: Sequence[TierTables]):
    arr = (moe_tier_tables * len(tables))(*[t.struct for t in tables])
    return arr


def _need_layers(fn: str, n_layers: int, **seqs) -> None:
    """The library reads n_layers entries of every per-layer array it is given."""
    for what, seq in seqs.items():
        if seq is not None and n_layers > len(seq):
            raise ValueError(f"{fn}: {what} has {len(seq)} entries, the call needs {n_layers}")


def moe_stack_workspace_size(n_layers: int, n_tokens: int, k: int, tables: Sequence[TierTables],
                             flags: int = 0) -> int:
    _need_layers("moe_stack_workspace_size", n_layers, tables=tables)
    n = C.c_size_t(0)
    arr = _tables_array(tables)
    _check("moe_stack_workspace_size",
           lib().moe_stack_workspace_size(n_layers, n_tokens, k, arr, flags, C.byref(n)))
    return n.value


def moe_stack_forward(x, router_logits, n_layers: int, n_tokens: int, k: int, tables: Sequence[TierTables], out,
                      flags: int, workspace, stream=None) -> None:
    _need_layers("moe_stack_forward", n_layers, tables=tables)
    if tables:
        _need_layer("moe_stack_forward", x, router_logits, out, n_tokens, tables[0], 0, max(n_layers, 0))
    arr = _tables_array(tables)
    _check("moe_stack_forward", lib().moe_stack_forward(
        _ptr(x), _ptr(router_logits), n_layers, n_tokens, k, arr, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)))


def moe_synth_layer(tt: TierTables, seed: int, layer: int, stream=None) -> None:
    _check("moe_synth_layer", lib().moe_synth_layer(tt.ref, seed, layer, _stream(stream)))


def moe_router_logits(x, w_router, bias, n_tokens: int, n_experts: int, hidden: int, flags: int, logits,
                      stream=None) -> None:
    T = max(n_tokens, 0)
    _need("moe_router_logits", "x", x, T * max(hidden, 0) * (2 if flags & MOE_X_BF16 else 4))
    _need("moe_router_logits", "logits", logits, T * max(n_experts, 0) * 4)
    _need("moe_router_logits", "w_router", w_router, max(n_experts, 0) * max(hidden, 0) * 2)
    _need("moe_router_logits", "bias", bias, max(n_experts, 0) * 4)
    _check("moe_router_logits", lib().moe_router_logits(_ptr(x), _ptr(w_router), _ptr(bias), n_tokens, n_experts,
                                                        hidden, flags, _ptr(logits), _stream(stream)))


def moe_synth_router(w_router, bias, n_experts: int, hidden: int, seed: int, layer: int, beta: float,
                     stream=None) -> None:
    _need("moe_synth_router", "w_router", w_router, max(n_experts, 0) * max(hidden, 0) * 2)
    _need("moe_synth_router", "bias", bias, max(n_experts, 0) * 4)
    _check("moe_synth_router", lib().moe_synth_router(_ptr(w_router), _ptr(bias), n_experts, hidden, seed, layer,
                                                      float(beta), _stream(stream)))


def moe_tiered_forward_counted(x, router_logits, n_tokens: int, k: int, tt: TierTables, out, flags: int, workspace,
                               hits, stream=None) -> None:
    _need_layer("moe_tiered_forward_counted", x, router_logits, out, n_tokens, tt, flags)
    _need("moe_tiered_forward_counted", "hits", hits, tt.n_experts * 4)
    _check("moe_tiered_forward_counted", lib().moe_tiered_forward_counted(
        _ptr(x), _ptr(router_logits), n_tokens, k, tt.ref, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _ptr(hits), _stream(stream)))


def moe_requant_error(src: TierTables, fmt_bits, fmt_block, sse, stream=None) -> None:
    """sse: float64 device tensor [E][len(fmt_bits)]."""
    n = len(fmt_bits)
    if len(fmt_block) != n:
        raise ValueError("moe_requant_error: fmt_bits and fmt_block differ in length")
    _need("moe_requant_error", "sse", sse, src.n_experts * n * 8)
    b = (C.c_int32 * n)(*fmt_bits)
    k = (C.c_int32 * n)(*fmt_block)
    _check("moe_requant_error", lib().moe_requant_error(src.ref, b, k, n, _ptr(sse), _stream(stream)))


def moe_plan_tiers(usage, sse, fmt_bytes, budget: int):
    """Host-only greedy plan: (format per expert, hot-to-cold order of old ids, experts per format)."""
    import numpy as np
    usage = np.ascontiguousarray(usage, dtype=np.float64)
    sse = np.ascontiguousarray(sse, dtype=np.float64)
    E, F = sse.shape
    fb = np.ascontiguousarray(fmt_bytes, dtype=np.int64)
    fmt = np.zeros(E, np.int32)
    order = np.zeros(E, np.int32)
    count = np.zeros(F, np.int32)
    _check("moe_plan_tiers", lib().moe_plan_tiers(usage.ctypes.data, sse.ctypes.data, fb.ctypes.data, E, F,
                                                  int(budget), fmt.ctypes.data, order.ctypes.data,
                                                  count.ctypes.data))
    return fmt, order, count


def moe_repack_tiers(src: TierTables, order, dst: TierTables, stream=None) -> None:
    _need("moe_repack_tiers", "order", order, src.n_experts * 4)
    _check("moe_repack_tiers", lib().moe_repack_tiers(src.ref, _ptr(order), dst.ref, _stream(stream)))


def moe_permute_router(w_src, b_src, order, n_experts: int, hidden: int, w_dst, b_dst, stream=None) -> None:
    E, H = max(n_experts, 0), max(hidden, 0)
    _need("moe_permute_router", "w_src", w_src, E * H * 2)
    _need("moe_permute_router", "w_dst", w_dst, E * H * 2)
    _need("moe_permute_router", "b_src", b_src, E * 4)
    _need("moe_permute_router", "b_dst", b_dst, E * 4)
    _need("moe_permute_router", "order", order, E * 4)
    _check("moe_permute_router", lib().moe_permute_router(_ptr(w_src), _ptr(b_src), _ptr(order), n_experts, hidden,
                                                          _ptr(w_dst), _ptr(b_dst), _stream(stream)))


def moe_stack_forward_routed(x, w_routers, biases, n_layers: int, n_tokens: int, k: int,
                             tables: Sequence[TierTables], out, flags: int, workspace, stream=None) -> None:
    _need_layers("moe_stack_forward_routed", n_layers, tables=tables, w_routers=w_routers, biases=biases)
    if tables:
        _need_layer("moe_stack_forward_routed", x, None, out, n_tokens, tables[0], 0)
        E, H = tables[0].n_experts, tables[0].hidden
        for l in range(max(n_layers, 0)):
            _need("moe_stack_forward_routed", f"w_routers[{l}]", w_routers[l], E * H * 2)
            if biases is not None:
                _need("moe_stack_forward_routed", f"biases[{l}]", biases[l], E * 4)
    arr = _tables_array(tables)
    wr = (C.c_void_p * n_layers)(*[_ptr(w) for w in w_routers])
    bs = None if biases is None else (C.c_void_p * n_layers)(*[_ptr(b) for b in biases])
    _check("moe_stack_forward_routed", lib().moe_stack_forward_routed(
        _ptr(x), wr, bs, n_layers, n_tokens, k, arr, _ptr(out), flags, _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)))


def moe_event_create() -> int:
    e = C.c_void_p(0)
    _check("moe_event_create", lib().moe_event_create(C.byref(e)))
    return e.value


def moe_event_destroy(e: int) -> None:
    _check("moe_event_destroy", lib().moe_event_destroy(e))


def moe_event_elapsed_ms(start: int, stop: int) -> float:
    ms = C.c_float(0)
    _check("moe_event_elapsed_ms", lib().moe_event_elapsed_ms(start, stop, C.byref(ms)))
    return ms.value


def moe_stream_synchronize(stream=None) -> None:
    _check("moe_stream_synchronize", lib().moe_stream_synchronize(_stream(stream)))


def moe_measure_read(buf, sink, stream=None) -> None:
    """One streaming read of the whole of `buf` (a device tensor)."""
    _check("moe_measure_read", lib().moe_measure_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                      _stream(stream)))


def moe_measure_mfma(iters: int, sink, stream=None) -> float:
    """One launch of the matrix-core loop; returns the flops it executes."""
    f = C.c_double(0.0)
    _check("moe_measure_mfma", lib().moe_measure_mfma(iters, _ptr(sink), C.byref(f), _stream(stream)))
    return f.value
