"""Parity of the raw-gate prologue and the conv state (through the C ABI) against the fp64 oracle.

Raw gates: the kernels receive a, b and gate_params = (A_log, dt_bias) and form g and beta
themselves; the oracle gets g and beta from its own fp64 gate function on the same fp32 inputs.
Conv state: a prefill reads the conv history before each sequence and leaves the last three raw
inputs; a decode step runs the conv on its token and shifts it in.  The history is a copy of
input values, so it must match the oracle's exactly.
"""
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


def _oracle_gates(a, b, gp):
    return oracle.gates(a, b, gp[0], gp[1])


def _prefill(wl, *, g, beta, gate_params=None, conv_state=None, segments=0, conv_fused=False):
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(g), TL.to_dev(beta),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), TL.to_dev(wl.conv_w), N=wl.N,
                          gate_params=TL.to_dev(gate_params), conv_state=conv_state, segments=segments,
                          conv_fused=conv_fused)
    torch.cuda.synchronize()
    return TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64)


def _oracle(wl, g, beta, hist=None):
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    return oracle.forward(wl.as_float("q"), wl.as_float("k"), wl.as_float("v"), g, beta, wl.s0, cu, wl.conv_w,
                          conv_hist=hist, want_conv_hist=wl.conv_w is not None)


# ------------------------------------------------------------------------------- raw gates

@pytest.mark.parametrize("dtype,dk,dv,conv", [("f32", 64, 32, False), ("f32", 32, 64, True),
                                              ("bf16", 128, 128, False), ("bf16", 64, 128, True)])
def test_raw_gates_prefill(dtype, dk, dv, conv):
    wl = W.make("raw_gates", seed=400 + dk + dv + conv, lengths=[130, 0, 64, 1, 77, 200], H=3, dk=dk, dv=dv,
                dtype=dtype, s0_std=0.05, conv=conv, varlen=True)
    a, b, gp = W.raw_gate_inputs(wl.meta["seed"], wl.lengths, wl.H)
    o, s = _prefill(wl, g=a, beta=b, gate_params=gp)
    g, beta = _oracle_gates(a, b, gp)
    o_ref, s_ref = _oracle(wl, g, beta)[:2]
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("raw_gates %s %d %d conv=%s %s" % (dtype, dk, dv, conv, e))


def test_raw_gates_prefill_segments():
    """The segmented long-sequence path with raw gates: every pass forms the gates itself."""
    wl = W.make("raw_gates_seg", seed=411, lengths=[64 * 40 + 17, 64 * 9], H=2, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, varlen=True)
    a, b, gp = W.raw_gate_inputs(wl.meta["seed"], wl.lengths, wl.H)
    g, beta = _oracle_gates(a, b, gp)
    o_ref, s_ref = _oracle(wl, g, beta)[:2]
    for segs in (1, 4):
        o, s = _prefill(wl, g=a, beta=b, gate_params=gp, segments=segs)
        e = TL.compare(wl, o, s, o_ref, s_ref)
        _flush("raw_gates segments=%d %s" % (segs, e))


def test_raw_gates_segments_slow_decay():
    """Raw gates with slow decay (A_log = log 1e-3, so g is about -1e-3 per token): no segment's
    transition is negligible, so the transition pass runs in full on its raw-gate instantiation
    (no output work), and the reruns cover whole segments."""
    wl = W.make("raw_gates_slow", seed=412, lengths=[64 * 12 + 9, 64 * 5], H=2, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, varlen=True)
    a, b, gp = W.raw_gate_inputs(wl.meta["seed"], wl.lengths, wl.H)
    gp = gp.copy()
    gp[0, :] = np.log(1e-3)
    g, beta = _oracle_gates(a, b, gp)
    assert g.max() < 0.0 and g.min() > -0.05, (g.min(), g.max())
    o_ref, s_ref = _oracle(wl, g, beta)[:2]
    o, s = _prefill(wl, g=a, beta=b, gate_params=gp, segments=3)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("raw_gates slow decay segments=3 %s" % e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_raw_gates_decode(dtype):
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    dw = W.decode(N=6, H=4, dk=128, dv=64, dtype=dtype, seed=421, state_std=0.3)
    a, b, gp = W.raw_gate_inputs(421, np.ones(dw.N, np.int64), dw.H)
    st = TL.to_dev(dw.state)
    o = gdn_recurrent_step(TL.to_dev(dw.q), TL.to_dev(dw.k), TL.to_dev(dw.v), TL.to_dev(a), TL.to_dev(b), st,
                           gate_params=TL.to_dev(gp))
    torch.cuda.synchronize()
    g, beta = _oracle_gates(a, b, gp)
    o_ref, s_ref = oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), g, beta, dw.state)
    _check_step(dtype, TL.o_to_f64(o), st.cpu().numpy().astype(np.float64), o_ref, s_ref)


def _check_step(dtype, og, sg, o_ref, s_ref):
    if dtype == "f32":
        assert np.abs(og - o_ref).max() / np.abs(o_ref).max() <= TL.F32_REL
        assert np.abs(sg - s_ref).max() / np.abs(s_ref).max() <= TL.F32_REL
    else:
        assert np.abs(og - o_ref).max() <= TL.BF16_O_ABS
        n = s_ref.shape[0] * s_ref.shape[1]
        d = np.linalg.norm((sg - s_ref).reshape(n, -1), axis=1)
        r = np.linalg.norm(s_ref.reshape(n, -1), axis=1)
        assert (d / r).max() <= TL.BF16_S_RELF


# ------------------------------------------------------------------------------ conv state

@pytest.mark.parametrize("dtype,dk,dv,fused", [("f32", 32, 64, False), ("bf16", 128, 128, False),
                                               ("bf16", 64, 32, False), ("bf16", 128, 64, True)])
def test_conv_state_prefill(dtype, dk, dv, fused):
    """History in, history out: sequences of 0, 1, 2 and 3 tokens keep part of the old history."""
    wl = W.make("conv_state", seed=430 + dk + dv, lengths=[130, 0, 1, 2, 3, 64, 77], H=2, dk=dk, dv=dv,
                dtype=dtype, s0_std=0.05, conv=True, varlen=True)
    _, hist = W.conv_inputs(wl.meta["seed"], wl.N, wl.H, dk, dv, dtype)
    cs = TL.to_dev(hist)
    o, s = _prefill(wl, g=wl.g, beta=wl.beta, conv_state=cs, conv_fused=fused)
    o_ref, s_ref, _, h_ref = _oracle(wl, wl.g, wl.beta, hist=W.bf16_bits_to_f32(hist) if dtype == "bf16" else hist)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    np.testing.assert_array_equal(_hist_to_f64(cs), h_ref)
    _flush("conv_state %s %d %d %s" % (dtype, dk, dv, e))


def test_conv_state_prefill_segments():
    """Segment 0 starts from the conv state, later segments from the tokens before them."""
    wl = W.make("conv_state_seg", seed=441, lengths=[64 * 36 + 5, 2], H=2, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, conv=True, varlen=True)
    _, hist = W.conv_inputs(441, wl.N, wl.H, 128, 128, "bf16")
    o_ref, s_ref, _, h_ref = _oracle(wl, wl.g, wl.beta, hist=W.bf16_bits_to_f32(hist))
    for segs in (1, 3):
        cs = TL.to_dev(hist)
        o, s = _prefill(wl, g=wl.g, beta=wl.beta, conv_state=cs, segments=segs)
        e = TL.compare(wl, o, s, o_ref, s_ref)
        np.testing.assert_array_equal(_hist_to_f64(cs), h_ref)
        _flush("conv_state segments=%d %s" % (segs, e))


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("f32", 32, 128), ("bf16", 128, 128), ("bf16", 128, 32)])
def test_conv_state_decode(dtype, dk, dv):
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    dw = W.decode(N=5, H=3, dk=dk, dv=dv, dtype=dtype, seed=450 + dk + dv, state_std=0.3)
    cw, hist = W.conv_inputs(450 + dk + dv, dw.N, dw.H, dk, dv, dtype)
    st, cs = TL.to_dev(dw.state), TL.to_dev(hist)
    o = gdn_recurrent_step(TL.to_dev(dw.q), TL.to_dev(dw.k), TL.to_dev(dw.v), TL.to_dev(dw.g), TL.to_dev(dw.beta),
                           st, conv_w=TL.to_dev(cw), conv_state=cs)
    torch.cuda.synchronize()
    h64 = W.bf16_bits_to_f32(hist) if dtype == "bf16" else hist
    o_ref, s_ref, h_ref = oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state,
                                      conv_w=cw, conv_hist=h64)
    _check_step(dtype, TL.o_to_f64(o), st.cpu().numpy().astype(np.float64), o_ref, s_ref)
    np.testing.assert_array_equal(_hist_to_f64(cs), h_ref)


@pytest.mark.parametrize("dtype,H,Hk", [("f32", 2, 2), ("bf16", 2, 2), ("f32", 4, 2), ("bf16", 6, 2)])
def test_prefill_split_then_decode_with_conv_and_raw_gates(dtype, H, Hk):
    """One sequence set fed as prefill(part 1) -> prefill(part 2) -> three decode steps, carrying
    the state and the conv state through the calls, with raw gates throughout, against the oracle
    over the whole sequences in one pass (also with value heads sharing query/key heads)."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd, gdn_recurrent_step
    import torch
    dk = dv = 64 if dtype == "f32" else 128
    lengths = [150, 71, 5]
    wl = W.make("pd_conv", seed=460 + H + Hk, lengths=lengths, H=H, Hk=Hk, dk=dk, dv=dv, dtype=dtype, s0_std=0.05,
                conv=True, varlen=True)
    a, b, gp = W.raw_gate_inputs(wl.meta["seed"], wl.lengths, wl.H)
    g, beta = _oracle_gates(a, b, gp)
    o_ref, s_ref, _, h_ref = _oracle(wl, g, beta)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    # token index sets: part 1 = first cut tokens, part 2 = up to the last 3, then 3 single steps
    cuts = [(int(cu[n]), int(cu[n]) + (L - 3) // 2, int(cu[n + 1]) - 3) for n, L in enumerate(lengths)]
    parts = [np.concatenate([np.arange(s, m) for s, m, _ in cuts]),
             np.concatenate([np.arange(m, e) for _, m, e in cuts])]
    dev = {name: TL.to_dev(getattr(wl, name)) for name in ("q", "k", "v")}
    da, db, dgp, dcw = TL.to_dev(a), TL.to_dev(b), TL.to_dev(gp), TL.to_dev(wl.conv_w)
    state = TL.to_dev(wl.s0)
    cs = torch.zeros((wl.N, 3, 2 * Hk * dk + H * dv), dtype=dev["q"].dtype, device=state.device)
    o_all = np.full((cu[-1], wl.H, dv), np.nan)
    for idx in parts:
        lens = [int(((idx >= cu[n]) & (idx < cu[n + 1])).sum()) for n in range(wl.N)]
        dcu = TL.to_dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        ti = torch.from_numpy(idx).cuda()
        o, state = gdn_chunk_fwd(*(dev[n][ti].contiguous() for n in ("q", "k", "v")), da[ti].contiguous(),
                                 db[ti].contiguous(), state, dcu, dcw, gate_params=dgp, conv_state=cs)
        torch.cuda.synchronize()
        o_all[idx] = TL.o_to_f64(o)
    for j in range(3):
        ti = torch.from_numpy(cu[1:] - 3 + j).cuda()
        o = gdn_recurrent_step(*(dev[n][ti].contiguous() for n in ("q", "k", "v")), da[ti].contiguous(),
                               db[ti].contiguous(), state, gate_params=dgp, conv_w=dcw, conv_state=cs)
        torch.cuda.synchronize()
        o_all[cu[1:] - 3 + j] = TL.o_to_f64(o)
    e = TL.compare(wl, o_all, state.cpu().numpy().astype(np.float64), o_ref, s_ref)
    np.testing.assert_array_equal(_hist_to_f64(cs), h_ref)
    _flush("prefill->prefill->decode conv+raw gates %s H=%d Hk=%d %s" % (dtype, H, Hk, e))
