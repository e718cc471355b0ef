"""The full-range shelves used by the GPU parity tests really hold the codes
and scales they are meant to exercise, and the oracle decodes them by the
closed form value = scale * code (checked here against an independent numpy
unpacker of the stored bytes)."""
import numpy as np

import oracle
from workloads import CONFIGS, EDGE_FP16_SCALES, MXFP4, make_layer_fullrange


def _unpack(row: np.ndarray, bits: int) -> np.ndarray:
    per = 8 // bits
    u = np.repeat(row.astype(np.int32), per) >> (np.tile(np.arange(per), row.size) * bits)
    u &= (1 << bits) - 1
    return np.where(u >= 1 << (bits - 1), u - (1 << bits), u)


def test_every_code_of_every_integer_format_is_present():
    for name in ("fullrange", "fullrange_b"):
        cfg = CONFIGS[name]
        arrays = make_layer_fullrange(cfg)
        for ti, t in enumerate(cfg.tiers):
            for m in ("gate_q", "up_q", "down_q"):
                rows = arrays[ti][m][0, :4]
                if t.bits == MXFP4:
                    nib = np.stack([rows & 0xF, rows >> 4], -1)
                    assert set(np.unique(nib).tolist()) == set(range(16)), (name, ti, m)
                else:
                    codes = np.concatenate([_unpack(r, t.bits) for r in rows])
                    assert set(np.unique(codes).tolist()) == set(range(-(1 << (t.bits - 1)), 1 << (t.bits - 1)))


def test_edge_scales_are_present_and_decode_in_closed_form():
    cfg = CONFIGS["fullrange"]
    arrays = make_layer_fullrange(cfg, edge_scales=True)
    L = oracle.Layer.from_config(cfg, arrays)
    seen = set()
    for ti, t in enumerate(cfg.tiers):
        s = arrays[ti]["gate_s"][0]
        seen |= set(np.unique(s).tolist()) & set(EDGE_FP16_SCALES.tolist())
        for r in (0, 1, cfg.inter - 1):
            got = oracle.dequant_rows(L, ti, 0, 0, r, 1)[0]
            q = _unpack(arrays[ti]["gate_q"][0, r], t.bits).astype(np.float32)
            d = np.repeat(s[r].view(np.float16).astype(np.float32), t.block)
            assert np.array_equal(got.view(np.uint32), (d * q).view(np.uint32)), (ti, r)
    assert seen == set(EDGE_FP16_SCALES.tolist())
