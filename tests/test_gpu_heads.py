"""Parity with value heads sharing query/key heads (H value heads, Hk query/key heads, value head h
reading query/key head h // (H // Hk)), through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

import gdn_testlib as TL
import oracle
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _hist_to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _run(wl, conv_state=None, segments=0):
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    cs = TL.to_dev(conv_state)
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(wl.g), TL.to_dev(wl.beta),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), TL.to_dev(wl.conv_w), N=wl.N,
                          conv_state=cs, segments=segments)
    torch.cuda.synchronize()
    return TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64), cs


def _oracle(wl, hist=None):
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    h64 = None if hist is None else (W.bf16_bits_to_f32(hist) if hist.dtype == np.uint16 else hist)
    return oracle.forward(wl.as_float("q"), wl.as_float("k"), wl.as_float("v"), wl.g, wl.beta, wl.s0, cu, wl.conv_w,
                          conv_hist=h64, want_conv_hist=wl.conv_w is not None)


@pytest.mark.parametrize("dtype,H,Hk,dk,dv,conv", [
    ("f32", 4, 2, 32, 64, True), ("f32", 3, 1, 64, 32, False),
    ("bf16", 4, 1, 128, 128, False), ("bf16", 6, 3, 64, 128, True), ("bf16", 8, 2, 128, 64, True),
])
def test_grouped_heads_prefill(dtype, H, Hk, dk, dv, conv):
    wl = W.make("gqa", seed=500 + H * 7 + Hk + dk + dv, lengths=[130, 0, 64, 1, 77, 200], H=H, Hk=Hk, dk=dk, dv=dv,
                dtype=dtype, s0_std=0.05, conv=conv, varlen=True)
    hist = W.conv_inputs(wl.meta["seed"], wl.N, H, dk, dv, dtype, Hk=Hk)[1] if conv else None
    o, s, cs = _run(wl, conv_state=hist)
    ref = _oracle(wl, hist)
    e = TL.compare(wl, o, s, ref[0], ref[1])
    if conv:
        np.testing.assert_array_equal(_hist_to_f64(cs), ref[3])
    _flush("gqa %s H=%d Hk=%d %d %d conv=%s %s" % (dtype, H, Hk, dk, dv, conv, e))


@pytest.mark.parametrize("slow", [False, True])
def test_grouped_heads_prefill_segments(slow):
    """Grouped heads on the segmented path; with `slow`, value head 1 (query/key head 0) decays at
    g = -1.5e-3, so its transitions are not negligible and the transition pass (which loads only
    the shared K) and full reruns run for it beside the fast heads."""
    wl = W.make("gqa_seg", seed=531, lengths=[64 * 40 + 9, 300], H=4, Hk=2, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, conv=True, varlen=True)
    if slow:
        wl.g[:, 1] = -1.5e-3
    hist = W.conv_inputs(531, wl.N, 4, 128, 128, "bf16", Hk=2)[1]
    ref = _oracle(wl, hist)
    for segs in (1, 4):
        o, s, cs = _run(wl, conv_state=hist, segments=segs)
        e = TL.compare(wl, o, s, ref[0], ref[1])
        np.testing.assert_array_equal(_hist_to_f64(cs), ref[3])
        _flush("gqa segments=%d slow=%s %s" % (segs, slow, e))


@pytest.mark.parametrize("dtype,H,Hk,dk,dv,conv", [
    ("f32", 4, 2, 64, 64, True), ("f32", 6, 1, 32, 128, False),
    ("bf16", 4, 2, 128, 128, True), ("bf16", 8, 4, 128, 32, False), ("bf16", 3, 3, 64, 64, True),
])
def test_grouped_heads_decode(dtype, H, Hk, dk, dv, conv):
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    seed = 540 + H + Hk + dk + dv
    dw = W.decode(N=5, H=H, Hk=Hk, dk=dk, dv=dv, dtype=dtype, seed=seed, state_std=0.3)
    cw, hist = W.conv_inputs(seed, dw.N, H, dk, dv, dtype, Hk=Hk) if conv else (None, None)
    st, cs = TL.to_dev(dw.state), TL.to_dev(hist)
    o = gdn_recurrent_step(TL.to_dev(dw.q), TL.to_dev(dw.k), TL.to_dev(dw.v), TL.to_dev(dw.g), TL.to_dev(dw.beta),
                           st, conv_w=TL.to_dev(cw), conv_state=cs)
    torch.cuda.synchronize()
    args = (dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state)
    if conv:
        h64 = W.bf16_bits_to_f32(hist) if dtype == "bf16" else hist
        o_ref, s_ref, h_ref = oracle.step(*args, conv_w=cw, conv_hist=h64)
        np.testing.assert_array_equal(_hist_to_f64(cs), h_ref)
    else:
        o_ref, s_ref = oracle.step(*args)
    og, sg = TL.o_to_f64(o), st.cpu().numpy().astype(np.float64)
    if dtype == "f32":
        assert np.abs(og - o_ref).max() / np.abs(o_ref).max() <= TL.F32_REL
        assert np.abs(sg - s_ref).max() / np.abs(s_ref).max() <= TL.F32_REL
    else:
        assert np.abs(og - o_ref).max() <= TL.BF16_O_ABS
        d = np.linalg.norm((sg - s_ref).reshape(dw.N * H, -1), axis=1)
        r = np.linalg.norm(s_ref.reshape(dw.N * H, -1), axis=1)
        assert (d / r).max() <= TL.BF16_S_RELF
