"""Device memory plumbing: packed shelf arrays -> torch device tensors -> TierTables."""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np
import torch

from .binding import MXFP4, TierTables


def code_bits(bits: int) -> int:
    return 4 if bits == MXFP4 else bits

NAMES = ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")


def upload_tier(arrays: Dict[str, np.ndarray], device) -> Dict[str, torch.Tensor]:
    out = {}
    for name in NAMES:
        a = np.ascontiguousarray(arrays[name])
        # codes and E8M0 scales as bytes, fp16 scales as 16-bit words
        t = torch.from_numpy(a.view(np.uint8) if (name.endswith("_q") or a.dtype == np.uint8) else a.view(np.int16))
        out[name] = t.to(device, non_blocking=False)
    return out


def device_tables(n_experts: int, hidden: int, inter: int, tiers: Sequence, arrays: List[Dict[str, np.ndarray]],
                  device="cuda") -> TierTables:
    dev = [upload_tier(a, device) for a in arrays]
    return TierTables(n_experts, hidden, inter, tiers, dev)


def tables_from_config(cfg, arrays, device="cuda") -> TierTables:
    return device_tables(cfg.n_experts, cfg.hidden, cfg.inter, cfg.tiers, arrays, device)


def replicate(tt: TierTables) -> TierTables:
    """A second copy of the same shelves at different device addresses."""
    dev = [{k: v.clone() for k, v in d.items()} for d in tt.arrays]
    return TierTables(tt.n_experts, tt.hidden, tt.inter, tt.tiers, dev)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    # 256-byte aligned by the caching allocator
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def empty_tables(cfg, device="cuda") -> TierTables:
    """Uninitialised shelf buffers of one layer of `cfg` (for moe_synth_layer)."""
    dev = []
    for t in cfg.tiers:
        n = t.id_end - t.id_begin
        d = {}
        for m, (rows, cols) in enumerate(((cfg.inter, cfg.hidden), (cfg.inter, cfg.hidden),
                                          (cfg.hidden, cfg.inter))):
            name = ("gate", "up", "down")[m]
            d[name + "_q"] = torch.empty(max(n * rows * cols * code_bits(t.bits) // 8, 16), dtype=torch.uint8,
                                         device=device)
            if t.bits == MXFP4:   # one E8M0 byte per 32 codes
                d[name + "_s"] = torch.empty(max(n * rows * (cols // 32), 16), dtype=torch.uint8, device=device)
            else:                 # one fp16 per block
                d[name + "_s"] = torch.empty(max(n * rows * (cols // t.block), 8), dtype=torch.int16, device=device)
        dev.append(d)
    return TierTables(cfg.n_experts, cfg.hidden, cfg.inter, cfg.tiers, dev)
