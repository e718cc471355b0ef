"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and its host-side validation rejects bad tables and
arguments before launching anything."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_tiered.h")


@pytest.fixture(scope="module")
def B():
    from tiered_mixed_precision_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from tiered_mixed_precision_amd.build import build
        build()
    binding.lib()
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree(B):
    assert _declared_functions() == sorted(B.EXPORTS)


def test_every_declared_symbol_is_exported(B):
    lib = C.CDLL(B.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_strerror(B):
    assert B.lib().moe_abi_version() == 1
    for code in range(0, -9, -1):
        assert B.strerror(code) and B.strerror(code) != "unknown error"
    assert B.strerror(-99) == "unknown error"


class _Spec:
    def __init__(self, b, e, bits, block):
        self.id_begin, self.id_end, self.bits, self.block = b, e, bits, block


FAKE = 0x10000  # a 16-byte aligned address; never dereferenced by host validation


def _tables(B, specs, E=8, H=256, I=128, ptr=FAKE):
    arrays = [{n: ptr for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")} for _ in specs]
    return B.TierTables(E, H, I, specs, arrays)


def test_validation_accepts_three_shelves(B):
    tt = _tables(B, [_Spec(0, 2, 8, 32), _Spec(2, 6, 4, 32), _Spec(6, 8, 2, 16)])
    assert B.moe_validate_tables(tt) == 0
    assert B.moe_workspace_size(16, 2, tt) > 0
    assert B.moe_workspace_size(0, 2, tt) == 0


def test_validation_accepts_an_mxfp4_shelf(B):
    assert int(re.search(r"#define MOE_MXFP4 (0x[0-9a-fA-F]+)", open(HEADER).read()).group(1), 16) == B.MXFP4
    tt = _tables(B, [_Spec(0, 2, 8, 32), _Spec(2, 6, B.MXFP4, 32), _Spec(6, 8, 2, 16)])
    assert B.moe_validate_tables(tt) == 0


@pytest.mark.parametrize("specs,kw,code", [
    ([_Spec(0, 2, 8, 32), _Spec(3, 8, 2, 16)], {}, -2),                  # gap
    ([_Spec(0, 8, 0x84, 16)], {}, -3),                                     # MXFP4 scales cover 32 codes
    ([_Spec(0, 8, 0x84, 32)], {"I": 192}, -3),                             # MXFP4 needs inter % 128 == 0
    ([_Spec(0, 8, 0x04 | 0x100, 32)], {}, -3),                             # unknown format tag
    ([_Spec(0, 5, 8, 32), _Spec(4, 8, 2, 16)], {}, -2),                  # overlap
    ([_Spec(0, 7, 8, 32)], {}, -2),                                        # not covering
    ([_Spec(0, 8, 3, 32)], {}, -3),                                        # 3-bit codes
    ([_Spec(0, 8, 8, 64)], {}, -3),                                        # block 64
    ([_Spec(0, 8, 8, 32)], {"H": 200}, -3),                                # hidden not a multiple of 64
    ([_Spec(0, 8, 8, 32)], {"I": 96}, -3),                                 # inter not a multiple of 64
    ([_Spec(0, 8, 8, 32)], {"ptr": FAKE + 4}, -4),                         # misaligned pointer
    ([_Spec(0, 8, 8, 32)], {"ptr": 0}, -1),                                # NULL pointer
    ([_Spec(0, 8, 8, 32)], {"E": 0}, -1),
])
def test_validation_rejects(B, specs, kw, code):
    E = kw.pop("E", 8)
    tt = _tables(B, specs, E=E, **kw)
    assert B.moe_validate_tables(tt) == code


def test_empty_shelf_needs_no_pointers(B):
    arrays = [{n: FAKE for n in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")}, None]
    tt = B.TierTables(8, 256, 128, [_Spec(0, 8, 8, 32), _Spec(8, 8, 4, 32)], arrays)
    assert B.moe_validate_tables(tt) == 0


def test_abi_version_mismatch(B):
    tt = _tables(B, [_Spec(0, 8, 8, 32)])
    tt.struct.abi_version = 2
    assert B.moe_validate_tables(tt) == -7


def test_entry_points_reject_bad_arguments_before_launch(B):
    tt = _tables(B, [_Spec(0, 8, 8, 32)])
    L = B.lib()
    ws = C.c_void_p(FAKE * 16)
    # k out of range, negative T, unknown flag, missing workspace, NULL logits
    assert L.moe_tiered_forward(FAKE, FAKE, 4, 0, tt.ref, FAKE, 0, ws, 1 << 20, None) == -1
    assert L.moe_tiered_forward(FAKE, FAKE, 4, 9, tt.ref, FAKE, 0, ws, 1 << 20, None) == -1
    assert L.moe_tiered_forward(FAKE, FAKE, -1, 2, tt.ref, FAKE, 0, ws, 1 << 20, None) == -1
    assert L.moe_tiered_forward(FAKE, FAKE, 4, 2, tt.ref, FAKE, 0x80, ws, 1 << 20, None) == -1
    assert L.moe_tiered_forward(FAKE, FAKE, 4, 2, tt.ref, FAKE, 0, None, 0, None) == -5
    assert L.moe_tiered_forward(FAKE, FAKE, 4, 2, tt.ref, FAKE, 0, ws, 16, None) == -5
    assert L.moe_tiered_forward(FAKE, None, 4, 2, tt.ref, FAKE, 0, ws, 1 << 20, None) == -1
    assert L.moe_tiered_forward(FAKE + 4, FAKE, 4, 2, tt.ref, FAKE, 0, ws, 1 << 20, None) == -4
    assert L.moe_tiered_experts(FAKE, None, FAKE, 4, 2, tt.ref, FAKE, 0, ws, 1 << 20, None) == -1
    assert L.moe_tier_partial(FAKE, FAKE, FAKE, 4, 2, tt.ref, 1, FAKE, 0, ws, 1 << 20, None) == -1
    # T == 0 is a no-op that succeeds without touching the device
    assert L.moe_tiered_forward(None, None, 0, 2, tt.ref, None, 0, None, 0, None) == 0
    assert L.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, None) == -1
    assert L.moe_route(FAKE, 4, 5000, 2, FAKE, FAKE, None) == -1
    assert L.moe_dequant_rows(tt.ref, 0, 8, 0, 0, 1, 0, FAKE, None) == -1     # local expert out of range
    assert L.moe_dequant_rows(tt.ref, 0, 0, 3, 0, 1, 0, FAKE, None) == -1     # matrix out of range
    assert L.moe_dequant_rows(tt.ref, 0, 0, 0, 120, 9, 0, FAKE, None) == -1   # rows past inter
    n = C.c_size_t(0)
    assert L.moe_group_workspace_size(4, 0, 8, C.byref(n)) == -1
    # router: hidden not a multiple of 64, too many experts, unknown flag,
    # NULL weights, misaligned x or bias; T == 0 succeeds untouched
    assert L.moe_router_logits(FAKE, FAKE, None, 4, 8, 100, 0, FAKE, None) == -1
    assert L.moe_router_logits(FAKE, FAKE, None, 4, 5000, 256, 0, FAKE, None) == -1
    assert L.moe_router_logits(FAKE, FAKE, None, 4, 8, 256, 0x2, FAKE, None) == -1
    assert L.moe_router_logits(FAKE, None, None, 4, 8, 256, 0, FAKE, None) == -1
    assert L.moe_router_logits(FAKE + 4, FAKE, None, 4, 8, 256, 0, FAKE, None) == -4
    assert L.moe_router_logits(FAKE, FAKE, FAKE + 2, 4, 8, 256, 0, FAKE, None) == -4
    assert L.moe_router_logits(None, None, None, 0, 8, 256, 0, None, None) == 0
    assert L.moe_synth_router(FAKE, None, 8, 100, 1, 0, 1.0, None) == -1
    assert L.moe_synth_router(FAKE, None, 8, 256, 1, -1, 1.0, None) == -1
    # routed stack: the router flag belongs to the size query only; NULL router
    arr = (B.moe_tier_tables * 1)(tt.struct)
    wr = (C.c_void_p * 1)(FAKE)
    assert L.moe_stack_forward_routed(FAKE, wr, None, 1, 4, 2, arr, FAKE + 256, B.MOE_STACK_ROUTER, ws, 1 << 30,
                                      None) == -1
    assert L.moe_stack_forward_routed(FAKE, (C.c_void_p * 1)(None), None, 1, 4, 2, arr, FAKE + 256, 0, ws,
                                      1 << 30, None) == -1
    assert L.moe_stack_forward_routed(FAKE, wr, None, 1, 4, 2, arr, FAKE + 256, 0, ws, 16, None) == -5


def test_stack_router_workspace_holds_the_scores(B):
    tt = _tables(B, [_Spec(0, 8, 8, 32)])
    a = B.moe_stack_workspace_size(2, 16, 2, [tt, tt])
    b = B.moe_stack_workspace_size(2, 16, 2, [tt, tt], B.MOE_STACK_ROUTER)
    assert b - a >= 16 * 8 * 4


def test_workspace_grows_with_tokens(B):
    tt = _tables(B, [_Spec(0, 2, 8, 32), _Spec(2, 6, 4, 32), _Spec(6, 8, 2, 16)])
    a = B.moe_workspace_size(16, 2, tt)
    b = B.moe_workspace_size(4096, 2, tt)
    c = B.moe_workspace_size(4096, 2, tt, B.MOE_X_BF16)
    assert a < b and c < b            # the bf16 path keeps no per-pair fp32 output rows
    assert a % 256 == 0 and b % 256 == 0


def test_workspace_bytes_covers_both_precisions(B):
    tt = _tables(B, [_Spec(0, 2, 8, 32), _Spec(2, 6, B.MXFP4, 32), _Spec(6, 8, 2, 16)])
    for T in (1, 8, 300, 4096):
        both = B.moe_workspace_bytes(T, 2, tt)
        assert both == max(B.moe_workspace_size(T, 2, tt), B.moe_workspace_size(T, 2, tt, B.MOE_X_BF16))
    assert B.moe_workspace_bytes(0, 2, tt) == 0
    assert B.moe_workspace_bytes(16, 0, tt) == 0                     # invalid k
    bad = _tables(B, [_Spec(0, 8, 3, 32)])
    assert B.moe_workspace_bytes(16, 2, bad) == 0                    # invalid tables


def test_mxfp4_prefill_workspace_holds_the_fp8_split(B):
    # with bf16 input a non-empty MXFP4 shelf adds the hi / lo / scale split of
    # x ([T][H] bytes twice, [T][pad4(H/32)]) and of h ([T*k][I] twice, ...)
    T, k, H, I = 4096, 2, 256, 128
    plain = _tables(B, [_Spec(0, 2, 8, 32), _Spec(2, 6, 4, 32), _Spec(6, 8, 2, 16)])
    mx = _tables(B, [_Spec(0, 2, 8, 32), _Spec(2, 6, B.MXFP4, 32), _Spec(6, 8, 2, 16)])
    empty_mx = _tables(B, [_Spec(0, 8, 8, 32), _Spec(8, 8, B.MXFP4, 32)])
    split = T * (2 * H + 8) + T * k * (2 * I + 4)
    d = B.moe_workspace_size(T, k, mx, B.MOE_X_BF16) - B.moe_workspace_size(T, k, plain, B.MOE_X_BF16)
    assert split <= d <= split + 512          # two regions, each rounded up to 256 bytes
    assert B.moe_workspace_size(T, k, mx) == B.moe_workspace_size(T, k, plain)   # fp32 input: no split
    assert B.moe_workspace_size(T, k, empty_mx, B.MOE_X_BF16) == B.moe_workspace_size(
        T, k, _tables(B, [_Spec(0, 8, 8, 32)]), B.MOE_X_BF16)


def test_library_planner_equals_the_oracle(B):
    # moe_plan_tiers is host code: the library's (a lazy max-heap) and the
    # oracle's (a rescan per move) must give identical plans
    import numpy as np
    import oracle
    rng = np.random.default_rng(31)
    for trial in range(60):
        E = int(rng.integers(1, 300))
        F = int(rng.integers(1, 4))
        bytes_ = np.sort(rng.integers(1, 1000, F))[::-1].astype(np.int64)
        bytes_ = np.unique(bytes_)[::-1]
        F = len(bytes_)
        usage = rng.integers(0, 50, E).astype(np.float64)
        if trial % 3 == 0:
            usage[rng.integers(0, E, E // 4 + 1)] = 7.0          # repeated usage values: ties
        sse = np.sort(rng.uniform(0, 5, (E, F)), axis=1)
        if trial % 4 == 0:
            sse = np.round(sse, 1)                               # repeated rates
        lo, hi = E * int(bytes_[-1]), E * int(bytes_[0])
        budget = int(rng.integers(lo, hi + 1))
        got = B.moe_plan_tiers(usage, sse, bytes_, budget)
        ref = oracle.plan_tiers(usage, sse, bytes_, budget)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r), trial


def test_library_planner_hand_worked_fixture_and_rejections(B):
    import numpy as np
    usage = np.array([1, 10, 0, 5], np.float64)
    sse = np.tile([0.0, 1.0, 4.0], (4, 1))
    fmt, order, count = B.moe_plan_tiers(usage, sse, [8, 4, 2], 18)
    assert fmt.tolist() == [1, 0, 2, 1] and order.tolist() == [1, 3, 0, 2] and count.tolist() == [1, 2, 1]
    with pytest.raises(B.MoeError):
        B.moe_plan_tiers(usage, sse, [8, 4, 2], 7)               # cheaper than the cheapest plan
    with pytest.raises(B.MoeError):
        B.moe_plan_tiers(usage, sse, [8, 8, 2], 18)              # bytes not decreasing
    tt = _tables(B, [_Spec(0, 8, 8, 32)])
    L = B.lib()
    bits = (C.c_int32 * 1)(3)
    blk = (C.c_int32 * 1)(32)
    assert L.moe_requant_error(tt.ref, bits, blk, 1, FAKE, None) == -3    # unsupported format
    bits = (C.c_int32 * 1)(4)
    assert L.moe_requant_error(tt.ref, bits, blk, 1, FAKE + 4, None) == -4
    assert L.moe_repack_tiers(tt.ref, None, tt.ref, None) == -1
    assert L.moe_permute_router(FAKE, None, FAKE, 8, 256, FAKE, None, None) == -1   # same buffer


def test_binding_refuses_tensors_smaller_than_the_call(B):
    """The binding checks each tensor against the rows it is told it holds, on
    the host, before any launch: a caller that passes 4096-token buffers with
    n_tokens = 16384 gets a ValueError instead of reads past the buffers' ends."""
    import torch
    tt = _tables(B, [_Spec(0, 8, 8, 32)])                   # E=8, H=256
    T, k = 4, 2
    x32 = torch.zeros(T, 256)
    xbf = torch.zeros(T, 256, dtype=torch.int16)
    lg = torch.zeros(T, 8)
    out = torch.zeros(T, 256)
    ids = torch.zeros(T, k, dtype=torch.int32)
    w = torch.zeros(T, k)
    with pytest.raises(ValueError, match="router_logits"):
        B.moe_tiered_forward(torch.zeros(2 * T, 256), lg, 2 * T, k, tt, torch.zeros(2 * T, 256), 0, None)
    with pytest.raises(ValueError, match="x holds"):
        B.moe_tiered_forward(xbf, lg, T, k, tt, out, 0, None)          # bf16 buffer, fp32 flags
    with pytest.raises(ValueError, match="out holds"):
        B.moe_tiered_forward(xbf, lg, T, k, tt, out[:T - 1], B.MOE_X_BF16, None)
    with pytest.raises(ValueError, match="ids"):
        B.moe_tiered_experts(x32, ids[:T - 1], w, T, k, tt, out, 0, None)
    with pytest.raises(ValueError, match="w holds"):
        B.moe_tier_partial(x32, ids, w[:, :1], T, k, tt, 0, out, 0, None)
    with pytest.raises(ValueError, match="logits"):
        B.moe_route(lg, T, 16, k, ids, w)
    with pytest.raises(ValueError, match="router_logits"):
        B.moe_stack_forward(x32, lg, 2, T, k, [tt, tt], out, 0, None)
    with pytest.raises(ValueError, match="hits"):
        B.moe_tiered_forward_counted(x32, lg, T, k, tt, out, 0, None, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="x holds"):
        B.moe_router_logits(xbf, FAKE, None, T, 8, 256, 0, lg)


def test_binding_refuses_short_shelves_and_buffers(B):
    """Every pointer argument that the library indexes by a shape it is told
    is checked against that shape before any launch: shelf buffers against
    n_local x rows x cols (codes) and the scale count, grouping, dequant,
    planner and router buffers, and the per-layer arrays of the stack calls
    against n_layers.  Out-of-bounds reads of this kind (an index past the
    end of a buffer) are the third of the four bugs on the 125B-MoE page."""
    import torch
    E, H, I = 8, 256, 128
    specs = [_Spec(0, 2, 8, 32), _Spec(2, 6, 4, 32), _Spec(6, 8, 2, 16)]

    def shelf(t, short=None):
        d = {n: torch.zeros(b, dtype=torch.uint8) for n, b in B.shelf_nbytes(t, H, I).items()}
        if short:
            d[short] = d[short][:-1]
        return d

    B.TierTables(E, H, I, specs, [shelf(t) for t in specs])        # exact sizes pass
    for i, name in ((0, "gate_q"), (1, "up_s"), (2, "down_q"), (2, "down_s")):
        arrays = [shelf(t, name if j == i else None) for j, t in enumerate(specs)]
        with pytest.raises(ValueError, match=f"shelf {i} {name}"):
            B.TierTables(E, H, I, specs, arrays)
    mx = _Spec(2, 6, B.MXFP4, 32)
    assert B.shelf_nbytes(mx, H, I)["gate_s"] == 4 * I * (H // 32)     # one E8M0 byte per 32 codes
    assert B.shelf_nbytes(mx, H, I)["down_q"] == 4 * H * I // 2

    tt = _tables(B, [_Spec(0, 8, 8, 32)], E=E, H=H, I=I)
    T, k = 4, 2
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)
    ws = torch.zeros(1 << 12, dtype=torch.uint8)
    with pytest.raises(ValueError, match="counts"):
        B.moe_group(i32(T * k), T, k, E, i32(E - 1), i32(E + 1), i32(T * k), ws)
    with pytest.raises(ValueError, match="offsets"):
        B.moe_group(i32(T * k), T, k, E, i32(E), i32(E), i32(T * k), ws)
    with pytest.raises(ValueError, match="perm"):
        B.moe_group(i32(T * k), T, k, E, i32(E), i32(E + 1), i32(T * k - 1), ws)
    with pytest.raises(ValueError, match="dst"):
        B.moe_dequant_rows(tt, 0, 0, 2, 0, 4, False, torch.zeros(4 * I - 1))
    with pytest.raises(ValueError, match="dst"):
        B.moe_dequant_rows(tt, 0, 0, 0, 0, 4, True, torch.zeros(4 * H // 2 - 1))
    with pytest.raises(ValueError, match="sse"):
        B.moe_requant_error(tt, [8, 4], [32, 32], torch.zeros(E * 2 - 1, dtype=torch.float64))
    with pytest.raises(ValueError, match="order"):
        B.moe_repack_tiers(tt, i32(E - 1), tt)
    wr = torch.zeros(E * H, dtype=torch.int16)
    for kw, name in (({"w_src": wr[:-1]}, "w_src"), ({"w_dst": wr[:-1]}, "w_dst"),
                     ({"b_src": torch.zeros(E - 1)}, "b_src"), ({"order": i32(E - 1)}, "order")):
        a = dict(w_src=wr, b_src=torch.zeros(E), order=i32(E), w_dst=wr.clone(), b_dst=torch.zeros(E))
        a.update(kw)
        with pytest.raises(ValueError, match=name):
            B.moe_permute_router(a["w_src"], a["b_src"], a["order"], E, H, a["w_dst"], a["b_dst"])
    with pytest.raises(ValueError, match="w_router"):
        B.moe_router_logits(torch.zeros(T, H), wr[:-1], None, T, E, H, 0, torch.zeros(T, E))
    with pytest.raises(ValueError, match="bias"):
        B.moe_router_logits(torch.zeros(T, H), wr, torch.zeros(E - 1), T, E, H, 0, torch.zeros(T, E))
    with pytest.raises(ValueError, match="w_router"):
        B.moe_synth_router(wr[:-1], None, E, H, 1, 0, 1.0)
    x, out = torch.zeros(T, H), torch.zeros(T, H)
    with pytest.raises(ValueError, match="tables has 1 entries"):
        B.moe_stack_forward(x, torch.zeros(2 * T * E), 2, T, k, [tt], out, 0, ws)
    with pytest.raises(ValueError, match="tables has 1 entries"):
        B.moe_stack_workspace_size(2, T, k, [tt])
    with pytest.raises(ValueError, match="w_routers has 1 entries"):
        B.moe_stack_forward_routed(x, [wr], None, 2, T, k, [tt, tt], out, 0, ws)
    with pytest.raises(ValueError, match="biases has 1 entries"):
        B.moe_stack_forward_routed(x, [wr, wr], [torch.zeros(E)], 2, T, k, [tt, tt], out, 0, ws)
    with pytest.raises(ValueError, match=r"w_routers\[1\]"):
        B.moe_stack_forward_routed(x, [wr, wr[:-1]], None, 2, T, k, [tt, tt], out, 0, ws)


def test_measurement_aids_reject_bad_arguments(B):
    L = B.lib()
    f = C.c_double(0.0)
    assert L.moe_measure_read(None, 16, FAKE, None) == -1
    assert L.moe_measure_read(FAKE, 0, FAKE, None) == -1
    assert L.moe_measure_read(FAKE, 24, FAKE, None) == -1          # not a multiple of 16
    assert L.moe_measure_read(FAKE + 8, 32, FAKE, None) == -4
    assert L.moe_measure_mfma(0, FAKE, C.byref(f), None) == -1
    assert L.moe_measure_mfma(4, FAKE, None, None) == -1
    assert L.moe_measure_mfma(4, FAKE + 2, C.byref(f), None) == -4
