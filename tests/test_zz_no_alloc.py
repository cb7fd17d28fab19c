"""gdn_chunk_fwd_noalloc against gdn_chunk_fwd: the entry point for callers that cannot allocate uses
the library's static scratch as its workspace and must give bitwise the results of the entry point
with a caller-provided workspace.  Two calls in a row, the second smaller, so the second runs on
scratch the first left behind: the segmented long-sequence path with a slowly decaying head
(transitions, chained entering states), then a 64-wide shape whose conv prologue runs as a
separate pass into the workspace.  Plus the same calls against the fp64 oracle.
"""
import numpy as np
import pytest

import gdn_testlib as TL
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    import torch
    assert a.shape == b.shape, what
    va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
    vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
    assert torch.equal(va, vb), what


def _both(wl, segments, **kw):
    import torch
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd, gdn_chunk_fwd_noalloc, gdn_chunk_workspace_size
    q, k, v, g, b = (TL.to_dev(x) for x in (wl.q, wl.k, wl.v, wl.g, wl.beta))
    s0, cu, cw = TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), TL.to_dev(wl.conv_w)
    need = gdn_chunk_workspace_size(wl.N, wl.T_tot, wl.H, wl.dk, wl.dv, has_cu_seqlens=cu is not None,
                                    has_conv=cw is not None,
                                    flags=1 | ((segments & 0xFF) << 8))
    assert need > 0, "the case must need a workspace"
    o_ref, s_ref = gdn_chunk_fwd(q, k, v, g, b, s0, cu, cw, N=wl.N, segments=segments, **kw)
    o = torch.empty_like(o_ref)
    sf = torch.empty_like(s_ref)
    gdn_chunk_fwd_noalloc(q, k, v, g, b, s0, cu, cw, N=wl.N, o=o, final_state=sf, segments=segments, **kw)
    torch.cuda.synchronize()
    _same(o, o_ref, "o, static scratch vs workspace")
    _same(sf, s_ref, "final state, static scratch vs workspace")
    return need, o, sf


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: segmented path, 2 sequences x 4 segments x 8 heads, head 1 decays slowly
    wl = W.make("noalloc_seg", seed=700, N=2, T=2048, H=8, dk=128, dv=128, dtype="bf16", s0_std=0.02)
    wl.g[:, 1] = -1e-3
    need1, o, sf = _both(wl, 4)
    o_ref, s_ref = TL.run_oracle(wl)
    e1 = TL.compare(wl, TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64), o_ref, s_ref)
    # second call, smaller, on the scratch the first one left: 64-wide heads with the conv pass in
    # the workspace, segments, varlen
    wl2 = W.make("noalloc_conv", seed=701, lengths=[300, 0, 700], H=2, dk=64, dv=64, dtype="bf16", s0_std=0.05,
                 conv=True, varlen=True)
    need2, o2, sf2 = _both(wl2, 3)
    assert need2 < need1
    o_ref2, s_ref2 = TL.run_oracle(wl2)
    e2 = TL.compare(wl2, TL.o_to_f64(o2), sf2.cpu().numpy().astype(np.float64), o_ref2, s_ref2)
    print("noalloc: workspace %d then %d bytes; %s; %s" % (need1, need2, e1, e2), flush=True)


def test_noalloc_too_large_is_rejected():
    """A call beyond the scratch is refused with GDN_ERR_SCRATCH, nothing launched (the outputs keep
    their sentinel)."""
    import torch
    from linear_attention_sequence_rule_amd import (GDN_ERR_SCRATCH, GDN_NOALLOC_SCRATCH_BYTES, GdnError,
                                                     gdn_chunk_fwd_noalloc, gdn_chunk_workspace_size)
    T, H, dk, dv = 1 << 17, 32, 64, 64
    assert gdn_chunk_workspace_size(1, T, H, dk, dv, has_cu_seqlens=False, has_conv=True,
                                    flags=1 | (1 << 8)) > GDN_NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    q = torch.zeros((T, H, dk), dtype=torch.bfloat16, device=dev)
    v = torch.zeros((T, H, dv), dtype=torch.bfloat16, device=dev)
    g = torch.zeros((T, H), dtype=torch.float32, device=dev)
    cw = torch.zeros((2 * H * dk + H * dv, 4), dtype=torch.float32, device=dev)
    o = torch.full((T, H, dv), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(GdnError) as ei:
        gdn_chunk_fwd_noalloc(q, q.clone(), v, g, g.clone(), None, None, cw, N=1, o=o, final_state=None, segments=1)
    assert ei.value.status == GDN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
