"""The allocation-free forward (engram_forward_noalloc) against engram_forward.

The allocation-free entry point runs the same kernels on the library's
static device workspace instead of a caller-provided one, so its highway must
equal engram_forward's bit for bit -- here on two calls in a row, the second
with fewer tokens, so that the second call runs on whatever the first left in
the static array.  Both are also held to the oracle on the small call.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.device import to_device, tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eg():
    import __graft_entry__
    __graft_entry__._ensure_built()
    import gram_hash_memory_amd
    torch.cuda.set_device(0)
    return gram_hash_memory_amd


def _objs(eg, wl, dw, T=None):
    """Binding objects for the first T tokens (whole sequences) of a workload."""
    s = wl.spec
    n_seqs = len(s.seq_lens)
    cu = wl.cu_seqlens
    if T is not None:
        n_seqs = int(np.searchsorted(cu, T))
        assert cu[n_seqs] == T
    cu_d = dw.cu_seqlens[:n_seqs + 1].contiguous()
    Tn = int(cu[n_seqs])
    lb = None if dw.lookback is None else dw.lookback[:n_seqs].contiguous()
    lbl = None if dw.lookback_live is None else dw.lookback_live[:n_seqs].contiguous()
    mask = None if dw.token_mask is None else dw.token_mask[:Tn].contiguous()
    docs = None if dw.doc_ids is None else dw.doc_ids[:Tn].contiguous()
    tokens = eg.Tokens(dw.cids[:Tn].contiguous(), cu_d, docs, mask, lb, lbl)
    params = eg.HashParams.from_dict(wl.hash_params)
    fmt = eg.ENGRAM_ROWS_Q2K if s.fmt == "q2k" else eg.ENGRAM_ROWS_FP8_E4M3_E8M0
    layers = [eg.Layer(fmt, l.table, l.scales, l.wkv, l.q_weight, l.k_weight, s.hc, s.dim,
                       s.cols) for l in dw.layers]
    return params, tokens, layers, Tn


@pytest.mark.parametrize("c,T_small", [(1, 17), (0, 64)])
def test_noalloc_forward_equals_forward_twice(eg, c, T_small):
    wl = workloads.make_workload(c)
    s = wl.spec
    dw = to_device(wl, "cuda")
    for T in (None, T_small):                      # full batch, then a smaller one
        params, tokens, layers, Tn = _objs(eg, wl, dw, T)
        need = eg.engram_workspace_bytes(Tn, len(s.layer_ids), s.cols, s.hc, s.dim)
        assert need <= eg.FORWARD_NOALLOC_MAX_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        h_ref = dw.h[:Tn].clone()
        bad_ref = torch.zeros(1, dtype=torch.int32, device="cuda")
        eg.engram_forward(params, tokens, layers, h_ref, s.hc, s.dim, s.eps, s.clamp,
                          s.dot_scale, ws, bad_ref)
        h = dw.h[:Tn].clone()
        bad = torch.zeros(1, dtype=torch.int32, device="cuda")
        eg.engram_forward_noalloc(params, tokens, layers, h, s.hc, s.dim, s.eps, s.clamp,
                                  s.dot_scale, bad)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), h_ref.view(torch.int32)), (c, Tn)
        assert bad.item() == bad_ref.item() == 0
    # the smaller call against the oracle as well
    hp = wl.hash_params
    n_seqs = int(np.searchsorted(wl.cu_seqlens, Tn))
    want = oracle.forward(wl.h[:Tn], wl.cids[:Tn], wl.cu_seqlens[:n_seqs + 1], hp,
                          [l.as_dict() for l in wl.layers], s.eps, s.clamp, s.dot_scale,
                          lookback=None if wl.lookback is None else wl.lookback[:n_seqs],
                          lookback_live=None if wl.lookback_live is None
                          else wl.lookback_live[:n_seqs])
    err = np.abs(h.cpu().numpy() - want) / np.maximum(1.0, np.abs(want))
    assert err.max() <= 1e-2, err.max()
