"""The guarantees the C ABI header states beyond parity, checked bitwise on the GPU.

* final_state may alias initial_state exactly: the in-place state hand-off of page
  maplevalley.com.cn/news/1910399, section 3.1 (initial_state = prev_memory -> last_state).  Aliased
  and separate buffers must give bitwise-equal o and final states: on the single pass, on the
  segmented path with more workgroups than the chip holds at once (so they queue) and with a slowly
  decaying head (the final state is then chained), and on the fp32 path.
* Results are bitwise reproducible run to run (no atomics).
* A NaN in one (sequence, head) chain never reaches another: chains are independent (page
  pzsr.cn/news/750, section 1: chunks in parallel inside a chain, serial between chunks of one chain).
* Packed variable-length sequences give bitwise the results of one call per sequence.
* Causality: changing q, k, v of tokens after t leaves o of tokens <= t bitwise unchanged.
"""
import numpy as np
import pytest

import gdn_testlib as TL
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _dev(wl):
    return dict(q=TL.to_dev(wl.q), k=TL.to_dev(wl.k), v=TL.to_dev(wl.v), g=TL.to_dev(wl.g), beta=TL.to_dev(wl.beta),
                s0=TL.to_dev(wl.s0), cu=TL.to_dev(wl.cu_seqlens), cw=TL.to_dev(wl.conv_w))


def _call(d, wl, *, s0=None, final=None, segments=0, **kw):
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    o, sf = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0, d["cu"], d["cw"], N=wl.N,
                          final_state=final, segments=segments, **kw)
    torch.cuda.synchronize()
    return o, sf


def _same(a, b, what):
    import torch
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), what


# ------------------------------------------------------------------------------------ aliasing

ALIAS_CASES = [
    # name, workload kwargs, segments, slow-decay heads
    ("single_pass_wide", dict(N=3, T=700, H=4, dk=128, dv=128, dtype="bf16"), 1, []),
    ("single_pass_narrow", dict(N=3, T=300, H=4, dk=64, dv=64, dtype="bf16"), 1, []),
    # 4 sequences x 8 segments x 16 heads = 512 workgroups of 128 rows: more than the 256 compute
    # units hold at once (one such workgroup per unit), so segment 0 and the last segment of a head
    # need not run together
    ("segments_queued_wide", dict(N=4, T=1024, H=16, dk=128, dv=128, dtype="bf16"), 8, [3]),
    # 64-row workgroups: 2 sequences x 8 segments x 20 heads = 320 workgroups
    ("segments_queued_narrow", dict(N=2, T=1100, H=20, dk=128, dv=64, dtype="bf16"), 8, [0, 5]),
    ("f32", dict(N=2, T=300, H=3, dk=64, dv=64, dtype="f32"), 1, []),
]


@pytest.mark.parametrize("name,kw,segments,slow", ALIAS_CASES, ids=[c[0] for c in ALIAS_CASES])
def test_final_state_aliases_initial_state(name, kw, segments, slow):
    import torch
    wl = W.make("alias_" + name, seed=600 + len(name), s0_std=0.05, **kw)
    for h in slow:
        wl.g[:, h] = -1e-3  # slow decay: full transitions, the final state chained by the rerun
    d = _dev(wl)
    o_sep, s_sep = _call(d, wl, s0=d["s0"].clone(), final=torch.empty_like(d["s0"]), segments=segments)
    buf = d["s0"].clone()
    o_al, s_al = _call(d, wl, s0=buf, final=buf, segments=segments)
    assert s_al.data_ptr() == buf.data_ptr()
    _same(o_al, o_sep, "o, aliased vs separate state buffers")
    _same(s_al, s_sep, "final state, aliased vs separate state buffers")
    # and both are right
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, TL.o_to_f64(o_al), s_al.cpu().numpy().astype(np.float64), o_ref, s_ref)
    _flush("alias %s segments=%d %s" % (name, segments, e))


# -------------------------------------------------------------------------------- determinism

def test_bitwise_reproducible():
    """The prefill workload, a segmented slow-decay call and a varlen + conv call, each twice."""
    import torch
    cases = [(W.prefill(), 0),
             (W.make("det_seg", seed=611, N=1, T=2048, H=4, dk=128, dv=128, dtype="bf16", s0_std=0.02), 4),
             (W.varlen(lengths=[700, 64, 3, 1500], H=4), 0)]
    cases[1][0].g[:, 1] = -1e-3
    for wl, segs in cases:
        d = _dev(wl)
        o1, s1 = _call(d, wl, s0=d["s0"], segments=segs)
        o2, s2 = _call(d, wl, s0=d["s0"], segments=segs)
        _same(o1, o2, "o run to run (%s)" % wl.name)
        _same(s1, s2, "final state run to run (%s)" % wl.name)
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------- NaN isolation

@pytest.mark.parametrize("segments", [1, 3])
@pytest.mark.parametrize("where", ["v", "q"])
def test_nan_stays_in_its_chain(segments, where):
    """A NaN planted in v (or q) of one token of chain (n=1, h=2): every other chain's o and final
    state is bitwise the clean run's, and so is o of that chain before the NaN's chunk."""
    import torch
    wl = W.make("nan", seed=620, lengths=[500, 900, 130, 700], H=4, dk=128, dv=128, dtype="bf16", s0_std=0.02,
                varlen=True, conv=True)
    d = _dev(wl)
    o_c, s_c = _call(d, wl, s0=d["s0"], segments=segments)
    n, h, t_in = 1, 2, 450  # token 450 of sequence 1 lies in its chunk 7
    t = int(wl.cu_seqlens[n]) + t_in
    bad = dict(d)
    bad[where] = d[where].clone()
    bad[where][t, h, 5] = float("nan")
    o_n, s_n = _call(bad, wl, s0=d["s0"], segments=segments)
    assert torch.isnan(o_n[t:int(wl.cu_seqlens[n + 1]), h]).any(), "the planted NaN shows in its own chain"
    keep = torch.ones(o_c.shape[:2], dtype=torch.bool, device=o_c.device)
    chunk0 = int(wl.cu_seqlens[n]) + (t_in // 64) * 64
    keep[chunk0:int(wl.cu_seqlens[n + 1]), h] = False
    _same(o_n[keep], o_c[keep], "o outside the poisoned chain (and before its chunk)")
    sk = torch.ones(s_c.shape[:2], dtype=torch.bool, device=s_c.device)
    sk[n, h] = False
    _same(s_n[sk], s_c[sk], "final states of the other chains")
    # the conv mixes neighbouring tokens only within one channel of one head: with the NaN in q the
    # state of the poisoned chain itself is clean
    if where == "q":
        _same(s_n[n, h], s_c[n, h], "final state of the chain whose q held the NaN")


# ------------------------------------------------------------------ varlen = separate calls

@pytest.mark.parametrize("dtype,dk,dv,conv", [("bf16", 128, 128, True), ("bf16", 64, 32, False),
                                              ("bf16", 128, 64, True), ("f32", 64, 64, True)])
def test_packed_equals_separate_calls(dtype, dk, dv, conv):
    """One packed call over sequences of lengths 300, 0, 64, 1, 129, 700 equals one call per
    sequence, bitwise (single pass in both: segments = 1)."""
    import torch
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    lengths = [300, 0, 64, 1, 129, 700]
    wl = W.make("packed", seed=630 + dk + dv, lengths=lengths, H=3, dk=dk, dv=dv, dtype=dtype, s0_std=0.05,
                varlen=True, conv=conv)
    d = _dev(wl)
    o_p, s_p = _call(d, wl, s0=d["s0"], segments=1)
    cu = wl.cu_seqlens
    for n, L in enumerate(lengths):
        a, b = int(cu[n]), int(cu[n + 1])
        one = torch.tensor([0, L], dtype=torch.int32, device=d["q"].device)
        # fresh copies: a slice of the packed tensors need not be 16-byte aligned
        o1, s1 = gdn_chunk_fwd(d["q"][a:b].clone(), d["k"][a:b].clone(), d["v"][a:b].clone(),
                               d["g"][a:b].clone(), d["beta"][a:b].clone(), d["s0"][n:n + 1].clone(),
                               one, d["cw"], segments=1)
        torch.cuda.synchronize()
        _same(o1, o_p[a:b], "o of sequence %d, separate vs packed" % n)
        _same(s1[0], s_p[n], "final state of sequence %d, separate vs packed" % n)


# ---------------------------------------------------------------------------------- causality

@pytest.mark.parametrize("segments", [1, 2])
@pytest.mark.parametrize("t_cut", [100, 191, 255])
def test_causality(t_cut, segments):
    """q, k, v of tokens > t_cut redrawn: o of tokens <= t_cut bitwise unchanged (inside a chunk
    too: the masked intra-chunk products add exact zeros)."""
    import torch
    wl = W.make("causal", seed=640, N=2, T=1024, H=4, dk=128, dv=128, dtype="bf16", s0_std=0.02, conv=True)
    d = _dev(wl)
    o_a, _ = _call(d, wl, s0=d["s0"], segments=segments)
    other = W.make("causal2", seed=641, N=2, T=1024, H=4, dk=128, dv=128, dtype="bf16", conv=True)
    d2 = dict(d)
    for name in ("q", "k", "v"):
        x = d[name].clone()
        y = TL.to_dev(getattr(other, name))
        for n in range(2):
            x[n * 1024 + t_cut + 1:(n + 1) * 1024] = y[n * 1024 + t_cut + 1:(n + 1) * 1024]
        d2[name] = x
    o_b, _ = _call(d2, wl, s0=d["s0"], segments=segments)
    for n in range(2):
        a, b = n * 1024, n * 1024 + t_cut + 1
        _same(o_b[a:b], o_a[a:b], "o of tokens <= %d (sequence %d)" % (t_cut, n))
        assert not torch.equal(o_b[b:(n + 1) * 1024], o_a[b:(n + 1) * 1024])
