"""Copy a seeded workload to GPU tensors (plumbing: no arithmetic of the method).

bf16 arrays travel as int16 tensors holding the bf16 bits; byte arrays as
uint8; ids as int32; the highway as float32.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def tensor(a, device, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


@dataclass
class DeviceLayer:
    fmt: str
    table: torch.Tensor
    scales: torch.Tensor | None
    wkv: torch.Tensor
    q_weight: torch.Tensor
    k_weight: torch.Tensor


@dataclass
class DeviceWorkload:
    cids: torch.Tensor
    cu_seqlens: torch.Tensor
    doc_ids: torch.Tensor | None
    token_mask: torch.Tensor | None
    lookback: torch.Tensor | None
    lookback_live: torch.Tensor | None
    layers: list = field(default_factory=list)
    h: torch.Tensor | None = None


def to_device(wl, device="cuda", with_layers=True, with_h=True) -> DeviceWorkload:
    dw = DeviceWorkload(cids=tensor(wl.cids, device, torch.int32),
                        cu_seqlens=tensor(wl.cu_seqlens, device, torch.int32),
                        doc_ids=tensor(wl.doc_ids, device, torch.int32),
                        token_mask=tensor(wl.token_mask, device, torch.uint8),
                        lookback=tensor(wl.lookback, device, torch.int32),
                        lookback_live=tensor(wl.lookback_live, device, torch.uint8))
    if with_layers:
        for l in wl.layers:
            dw.layers.append(DeviceLayer(l.fmt, tensor(l.table, device),
                                         tensor(l.scales, device), tensor(l.wkv, device),
                                         tensor(l.q_weight, device), tensor(l.k_weight, device)))
    if with_h and wl.h is not None:
        dw.h = tensor(wl.h, device)
    return dw
