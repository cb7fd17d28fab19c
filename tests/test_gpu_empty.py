"""Calls whose every sequence is empty (T_tot = 0): the state passes through unchanged, the conv
history is kept as it was, and nothing else is touched.  The q, k, v, g, beta, o (and z) tensors
are empty, so their device pointers are null; no kernel may read a token.  Covered on the wide
kernel (with the fused conv, the output epilogue, and forced segments), the narrow kernel (with
the streaming conv pass) and the fp32 kernel, each checked bit for bit against the initial state
and history, and against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from linear_attention_sequence_rule_amd import workloads as W
import gdn_testlib as TL

pytestmark = pytest.mark.gpu


def _hist_to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,dk,dv,varlen,segments,state,epi", [
    ("bf16", 128, 128, True, 0, True, True),     # wide kernel, fused conv and epilogue
    ("bf16", 128, 128, False, 3, True, False),   # wide kernel, three forced (empty) segments
    ("bf16", 64, 32, True, 0, False, True),      # narrow kernel, streaming conv pass, separate epilogue
    ("f32", 64, 32, True, 0, True, False),       # fp32 kernel
])
def test_all_sequences_empty(dtype, dk, dv, varlen, segments, state, epi):
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    H, N = 2, 3
    print("empty %s dk=%d dv=%d varlen=%s segments=%d" % (dtype, dk, dv, varlen, segments), flush=True)
    wl = W.make("empty", seed=900 + dk + dv + segments, lengths=[0] * N, H=H, dk=dk, dv=dv, dtype=dtype,
                s0_std=0.05 if state else None, conv=True, varlen=varlen)
    _, hist = W.conv_inputs(wl.meta["seed"], N, H, dk, dv, dtype)
    cs = TL.to_dev(hist)
    z = TL.to_dev(np.zeros((0, H, dv), dtype=wl.v.dtype)) if epi else None
    nw = TL.to_dev(np.linspace(-0.5, 0.5, dv, dtype=np.float32)) if epi else None
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(wl.g), TL.to_dev(wl.beta),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), TL.to_dev(wl.conv_w), N=N, conv_state=cs,
                          out_gate=z, norm_weight=nw, segments=segments)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (0, H, dv)
    s = sf.cpu().numpy()
    want = wl.s0 if state else np.zeros((N, H, dv, dk), np.float32)
    np.testing.assert_array_equal(s, want)
    np.testing.assert_array_equal(_hist_to_f64(cs), _hist_to_f64(TL.to_dev(hist)))
    cu = np.zeros(N + 1, np.int64)
    _, s_ref, _, h_ref = oracle.forward(wl.as_float("q"), wl.as_float("k"), wl.as_float("v"), wl.g, wl.beta, wl.s0,
                                        cu, wl.conv_w, conv_hist=W.bf16_bits_to_f32(hist) if dtype == "bf16" else hist,
                                        want_conv_hist=True)
    np.testing.assert_array_equal(s.astype(np.float64), s_ref)
    np.testing.assert_array_equal(_hist_to_f64(cs), h_ref)


def test_decode_empty_batch():
    """N = 0 decode: a no-op that launches nothing and returns an empty output."""
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    H, dk, dv = 2, 128, 128
    e = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    f = lambda *shape: torch.zeros(shape, dtype=torch.float32, device="cuda")
    o = gdn_recurrent_step(e(0, H, dk), e(0, H, dk), e(0, H, dv), f(0, H), f(0, H), f(0, H, dv, dk))
    torch.cuda.synchronize()
    assert tuple(o.shape) == (0, H, dv)
