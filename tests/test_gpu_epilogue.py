"""Parity of the output epilogue (zero-centred RMSNorm over dv, then a sigmoid output gate) through
the C ABI against the fp64 oracle.

Tolerances.  fp32 paths: max|gpu - ref| / max|ref| <= 1e-4, as for o.  bf16 decode: o is formed in
fp32 inside the step kernel and rounded to bf16 once, after the epilogue: |gpu - ref| <= 2^-8 |ref|
+ 1e-5 elementwise.  bf16 prefill: the epilogue runs on the stored bf16 o, whose own bar is
max|do| <= 2e-2; to first order the normalisation maps an error do in a row to
m (do - o (o . do) / (dv ms)) / rms with m = (1 + w) sigmoid(z), which is at most 2 m max|do| / rms,
so the bar is |gpu - ref| <= 2 m 2e-2 / rms_ref + 2^-8 |ref| + 1e-5 per element, rms_ref the
oracle row's sqrt(mean o^2 + eps).  With dk = dv = 128 the chunk kernel applies the epilogue itself
to its fp32 o and rounds once; its o error before that rounding is below the bar of the stored
bf16 o, so the same bound holds.
"""
import numpy as np
import pytest

import gdn_testlib as TL
import oracle
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _epilogue_inputs(seed, rows_shape, dv, dtype):
    r = np.random.default_rng([seed, 77])
    z = r.standard_normal(rows_shape + (dv,), dtype=np.float32)
    w = r.normal(0.0, 0.2, size=dv).astype(np.float32)
    return (W.f32_to_bf16_bits(z) if dtype == "bf16" else z), w


def _zf(z):
    return W.bf16_bits_to_f32(z) if z.dtype == np.uint16 else z


@pytest.mark.parametrize("dtype,dk,dv,eps", [("f32", 32, 64, 1e-6), ("f32", 64, 32, 1e-3),
                                             ("bf16", 128, 128, 1e-3), ("bf16", 64, 32, 1e-6)])
def test_epilogue_prefill(dtype, dk, dv, eps):
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    wl = W.make("epi", seed=600 + dk + dv, lengths=[130, 0, 64, 1, 77], H=3, dk=dk, dv=dv, dtype=dtype,
                s0_std=0.05, varlen=True)
    z, w = _epilogue_inputs(wl.meta["seed"], (wl.T_tot, wl.H), dv, dtype)
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(wl.g), TL.to_dev(wl.beta),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), out_gate=TL.to_dev(z), norm_weight=TL.to_dev(w),
                          norm_eps=eps)
    torch.cuda.synchronize()
    og, sg = TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64)
    o_ref, s_ref = TL.run_oracle(wl)
    ref = oracle.gated_norm(o_ref, _zf(z), w, eps)
    # the state is untouched by the epilogue
    TL.compare(wl, o_ref, sg, o_ref, s_ref)
    if dtype == "f32":
        assert np.abs(og - ref).max() / np.abs(ref).max() <= TL.F32_REL
    else:
        m = (1.0 + w.astype(np.float64)) / (1.0 + np.exp(-_zf(z).astype(np.float64)))
        rms = np.sqrt((o_ref ** 2).mean(-1, keepdims=True) + eps)
        bound = 2 * m * TL.BF16_O_ABS / rms + 2.0 ** -8 * np.abs(ref) + 1e-5
        excess = np.abs(og - ref) / bound
        assert excess.max() <= 1.0, excess.max()
        _flush("epilogue prefill bf16 %d %d: max err %.3g, max err/bound %.3g" % (dk, dv, np.abs(og - ref).max(),
                                                                                   excess.max()))


def test_epilogue_prefill_segments_and_conv():
    """The epilogue after the segmented path with the conv prologue and grouped heads."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    wl = W.make("epi_seg", seed=611, lengths=[64 * 36 + 11, 5], H=4, Hk=2, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, conv=True, varlen=True)
    z, w = _epilogue_inputs(611, (wl.T_tot, wl.H), 128, "bf16")
    o, _ = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(wl.g), TL.to_dev(wl.beta),
                         TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), TL.to_dev(wl.conv_w), segments=3,
                         out_gate=TL.to_dev(z), norm_weight=TL.to_dev(w), norm_eps=1e-3)
    torch.cuda.synchronize()
    og = TL.o_to_f64(o)
    o_ref, _ = TL.run_oracle(wl)
    ref = oracle.gated_norm(o_ref, _zf(z), w, 1e-3)
    m = (1.0 + w.astype(np.float64)) / (1.0 + np.exp(-_zf(z).astype(np.float64)))
    rms = np.sqrt((o_ref ** 2).mean(-1, keepdims=True) + 1e-3)
    excess = np.abs(og - ref) / (2 * m * TL.BF16_O_ABS / rms + 2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 1.0, excess.max()
    _flush("epilogue segments+conv+groups: max err %.3g, max err/bound %.3g" % (np.abs(og - ref).max(), excess.max()))


def test_epilogue_prefill_output_scale():
    """The fused epilogue with a negative, non-unit output scale on the segmented path: the scale
    rides in the prepared output operands (also the kept ones the reruns use), and the norm sees
    the scaled o."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    wl = W.make("epi_scale", seed=613, lengths=[64 * 9 + 5, 64 * 3], H=3, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, varlen=True)
    z, w = _epilogue_inputs(613, (wl.T_tot, wl.H), 128, "bf16")
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(wl.g), TL.to_dev(wl.beta),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), segments=3, scale=-0.37, out_gate=TL.to_dev(z),
                          norm_weight=TL.to_dev(w), norm_eps=1e-3)
    torch.cuda.synchronize()
    og, sg = TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64)
    o_ref, s_ref = TL.run_oracle(wl, scale=-0.37)
    TL.compare(wl, o_ref, sg, o_ref, s_ref)
    ref = oracle.gated_norm(o_ref, _zf(z), w, 1e-3)
    m = (1.0 + w.astype(np.float64)) / (1.0 + np.exp(-_zf(z).astype(np.float64)))
    rms = np.sqrt((o_ref ** 2).mean(-1, keepdims=True) + 1e-3)
    excess = np.abs(og - ref) / (2 * m * TL.BF16_O_ABS / rms + 2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 1.0, excess.max()
    _flush("epilogue scale -0.37: max err %.3g, max err/bound %.3g" % (np.abs(og - ref).max(), excess.max()))


def test_epilogue_prefill_segments_grouped():
    """The epilogue on the segmented path without the conv, grouped heads: reruns whose first chunk
    reaches the decay bound redo only that chunk (one of them a partial chunk: the last segment of
    the 138-token sequence has 10 tokens), while head 3, slowly decaying, reruns in full."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    wl = W.make("epi_seg_gqa", seed=612, lengths=[64 * 30 + 17, 64 * 2 + 10, 40], H=4, Hk=2, dk=128, dv=128,
                dtype="bf16", s0_std=0.02, varlen=True)
    wl.g[:, 3] = -2e-3
    z, w = _epilogue_inputs(612, (wl.T_tot, wl.H), 128, "bf16")
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(wl.g), TL.to_dev(wl.beta),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), segments=3, out_gate=TL.to_dev(z),
                          norm_weight=TL.to_dev(w), norm_eps=1e-3)
    torch.cuda.synchronize()
    og, sg = TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64)
    o_ref, s_ref = TL.run_oracle(wl)
    TL.compare(wl, o_ref, sg, o_ref, s_ref)
    ref = oracle.gated_norm(o_ref, _zf(z), w, 1e-3)
    m = (1.0 + w.astype(np.float64)) / (1.0 + np.exp(-_zf(z).astype(np.float64)))
    rms = np.sqrt((o_ref ** 2).mean(-1, keepdims=True) + 1e-3)
    excess = np.abs(og - ref) / (2 * m * TL.BF16_O_ABS / rms + 2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 1.0, excess.max()
    _flush("epilogue segments+groups: max err %.3g, max err/bound %.3g" % (np.abs(og - ref).max(), excess.max()))


@pytest.mark.parametrize("dtype,H,Hk,dk,dv,conv", [("f32", 3, 3, 64, 64, False), ("f32", 4, 2, 32, 128, True),
                                                   ("bf16", 4, 4, 128, 128, False), ("bf16", 4, 2, 128, 128, True),
                                                   ("bf16", 2, 1, 64, 32, True)])
def test_epilogue_decode(dtype, H, Hk, dk, dv, conv):
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    seed = 620 + H + Hk + dk + dv
    dw = W.decode(N=6, H=H, Hk=Hk, dk=dk, dv=dv, dtype=dtype, seed=seed, state_std=0.3)
    z, w = _epilogue_inputs(seed, (dw.N, H), dv, dtype)
    cw, hist = W.conv_inputs(seed, dw.N, H, dk, dv, dtype, Hk=Hk) if conv else (None, None)
    st, cs = TL.to_dev(dw.state), TL.to_dev(hist)
    o = gdn_recurrent_step(TL.to_dev(dw.q), TL.to_dev(dw.k), TL.to_dev(dw.v), TL.to_dev(dw.g), TL.to_dev(dw.beta),
                           st, conv_w=TL.to_dev(cw), conv_state=cs, out_gate=TL.to_dev(z), norm_weight=TL.to_dev(w),
                           norm_eps=1e-3)
    torch.cuda.synchronize()
    args = (dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state)
    if conv:
        o_ref, s_ref, _ = oracle.step(*args, conv_w=cw, conv_hist=_zf(hist))
    else:
        o_ref, s_ref = oracle.step(*args)
    ref = oracle.gated_norm(o_ref, _zf(z), w, 1e-3)
    og, sg = TL.o_to_f64(o), st.cpu().numpy().astype(np.float64)
    if dtype == "f32":
        assert np.abs(og - ref).max() / np.abs(ref).max() <= TL.F32_REL
        assert np.abs(sg - s_ref).max() / np.abs(s_ref).max() <= TL.F32_REL
    else:
        assert (np.abs(og - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5).all(), np.abs(og - ref).max()
        d = np.linalg.norm((sg - s_ref).reshape(dw.N * H, -1), axis=1)
        r = np.linalg.norm(s_ref.reshape(dw.N * H, -1), axis=1)
        assert (d / r).max() <= TL.BF16_S_RELF


def test_epilogue_prefill_raw_gates_conv_history():
    """The epilogue in the 128-row kernel together with raw gates, the conv prologue on a conv
    history, grouped heads and forced segments (every input path the kernel has at once)."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    wl = W.make("epi_all", seed=621, lengths=[64 * 20 + 3, 70, 1], H=4, Hk=2, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, conv=True, varlen=True)
    a, b, gp = W.raw_gate_inputs(621, wl.lengths, wl.H)
    hist = W.conv_inputs(621, wl.N, wl.H, 128, 128, "bf16", Hk=2)[1]
    z, w = _epilogue_inputs(621, (wl.T_tot, wl.H), 128, "bf16")
    cs = TL.to_dev(hist)
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(a), TL.to_dev(b),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), TL.to_dev(wl.conv_w), N=wl.N,
                          gate_params=TL.to_dev(gp), conv_state=cs, segments=2, out_gate=TL.to_dev(z),
                          norm_weight=TL.to_dev(w), norm_eps=1e-3)
    torch.cuda.synchronize()
    og, sg = TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64)
    g, beta = oracle.gates(a, b, gp[0], gp[1])
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    o_ref, s_ref, _ = oracle.forward(wl.as_float("q"), wl.as_float("k"), wl.as_float("v"), g, beta, wl.s0, cu,
                                     wl.conv_w, conv_hist=_zf(hist))[:3]
    TL.compare(wl, o_ref, sg, o_ref, s_ref)
    ref = oracle.gated_norm(o_ref, _zf(z), w, 1e-3)
    m = (1.0 + w.astype(np.float64)) / (1.0 + np.exp(-_zf(z).astype(np.float64)))
    rms = np.sqrt((o_ref ** 2).mean(-1, keepdims=True) + 1e-3)
    excess = np.abs(og - ref) / (2 * m * TL.BF16_O_ABS / rms + 2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 1.0, excess.max()
    _flush("epilogue raw gates+conv history+groups+segments: max err %.3g, max err/bound %.3g"
           % (np.abs(og - ref).max(), excess.max()))


def test_epilogue_raw_gates_slow_decay_queued():
    """The transition and rerun passes in one launch on the instantiation with raw gates and the
    epilogue: 3 sequences x 8 segments x 16 value heads = 384 workgroups (more than the compute
    units hold at once) on 8 query/key heads, and every fourth head decaying slowly (A_log =
    log 1e-3, g about -1e-3 per token), so those transitions are formed in full and later reruns
    wait for them; the other heads' reruns redo one chunk from the kept operands."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    wl = W.make("epi_raw_slow", seed=631, N=3, T=1024, H=16, Hk=8, dk=128, dv=128, dtype="bf16", s0_std=0.02,
                varlen=True)
    a, b, gp = W.raw_gate_inputs(631, wl.lengths, wl.H)
    gp = gp.copy()
    gp[0, ::4] = np.log(1e-3)
    z, w = _epilogue_inputs(631, (wl.T_tot, wl.H), 128, "bf16")
    o, sf = gdn_chunk_fwd(TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v), TL.to_dev(a), TL.to_dev(b),
                          TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens), N=wl.N, gate_params=TL.to_dev(gp), segments=8,
                          out_gate=TL.to_dev(z), norm_weight=TL.to_dev(w), norm_eps=1e-3)
    torch.cuda.synchronize()
    og, sg = TL.o_to_f64(o), sf.cpu().numpy().astype(np.float64)
    g, beta = oracle.gates(a, b, gp[0], gp[1])
    assert g[:, ::4].min() > -0.05 and g[:, 1::4].mean() < -0.2
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    o_ref, s_ref, _ = oracle.forward(wl.as_float("q"), wl.as_float("k"), wl.as_float("v"), g, beta, wl.s0, cu)
    TL.compare(wl, o_ref, sg, o_ref, s_ref)
    ref = oracle.gated_norm(o_ref, _zf(z), w, 1e-3)
    m = (1.0 + w.astype(np.float64)) / (1.0 + np.exp(-_zf(z).astype(np.float64)))
    rms = np.sqrt((o_ref ** 2).mean(-1, keepdims=True) + 1e-3)
    excess = np.abs(og - ref) / (2 * m * TL.BF16_O_ABS / rms + 2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 1.0, excess.max()
    _flush("epilogue raw gates slow decay queued: max err %.3g, max err/bound %.3g" % (np.abs(og - ref).max(),
                                                                                      excess.max()))


# ------------------------------------------------ the epilogue against the norm of the kernel's own o

U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits, round to nearest even)

ROUNDING_CASES = [
    # name, workload kwargs, segments, fused (the 128-row kernel applies the epilogue to its fp32 o)
    ("prefill_bench_shape", None, 0, True),
    ("wide_conv_groups_segments", dict(lengths=[64 * 9 + 5, 130, 1], H=4, Hk=2, dk=128, dv=128, dtype="bf16",
                                       conv=True), 3, True),
    ("narrow_128x64", dict(lengths=[300, 64, 7], H=4, dk=128, dv=64, dtype="bf16"), 2, False),
    ("narrow_64x32_conv", dict(lengths=[200, 1, 90], H=3, dk=64, dv=32, dtype="bf16", conv=True), 0, False),
    ("f32_64x64", dict(lengths=[150, 33], H=3, dk=64, dv=64, dtype="f32"), 0, False),
]


@pytest.mark.parametrize("name,kw,segments,fused", ROUNDING_CASES, ids=[c[0] for c in ROUNDING_CASES])
def test_epilogue_is_the_norm_of_its_own_output(name, kw, segments, fused):
    """The same call with and without the epilogue: the gated output must be the fp64 gated norm of
    the un-gated output up to the roundings the path takes, a bar set by bf16 rounding alone rather
    than by the o parity bar.

    Fused (128-row kernel, bf16): the kernel normalises its fp32 o and rounds once, while the
    un-gated call rounds that same o to bf16.  A relative change of at most u = 2^-8 in every element
    of a row moves each o_i / rms by at most 2u |o_i| / rms to first order (u from o_i, u from rms), and
    the final rounding adds u: |gated - gated_norm(o_plain)| <= 3u |ref|.  Separate pass (other
    shapes, bf16): the norm reads the stored bf16 o, which is o_plain itself, and rounds once: u |ref|.
    fp32: the norm reads the stored fp32 o; only fp32 arithmetic separates them.  A relative 1e-5
    covers the fp32 arithmetic of the norm (rsqrt, exp, reciprocal) and an absolute 1e-6 of the row's
    largest value covers elements that cancel to ~0."""
    import torch
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    if kw is None:
        wl = W.prefill()
    else:
        wl = W.make("epi_round_" + name, seed=650 + len(name), s0_std=0.05, varlen=True, **kw)
    z, w = _epilogue_inputs(660 + len(name), (wl.T_tot, wl.H), wl.dv, wl.dtype)
    d = dict(q=TL.to_dev(wl.q), k=TL.to_dev(wl.k), v=TL.to_dev(wl.v), g=TL.to_dev(wl.g), beta=TL.to_dev(wl.beta),
             s0=TL.to_dev(wl.s0), cu=TL.to_dev(wl.cu_seqlens), cw=TL.to_dev(wl.conv_w))
    zd, wd = TL.to_dev(z), TL.to_dev(w)

    def run(gated):
        o, sf = gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["cu"], d["cw"], N=wl.N,
                              segments=segments, out_gate=zd if gated else None, norm_weight=wd if gated else None,
                              norm_eps=1e-3)
        torch.cuda.synchronize()
        return o, sf

    o_plain, s_plain = run(False)
    o_gated, s_gated = run(True)
    assert torch.equal(s_plain, s_gated), "the epilogue leaves the final state alone"
    og = TL.o_to_f64(o_gated)
    ref = oracle.gated_norm(TL.o_to_f64(o_plain), _zf(z), w, 1e-3)
    rel = (3 * U_BF16 if fused else U_BF16) if wl.dtype == "bf16" else 0.0
    bound = (rel + 1e-5) * np.abs(ref) + 1e-6 * np.abs(ref).max(-1, keepdims=True)
    excess = np.abs(og - ref) / bound
    _flush("epilogue rounding %s: max |err|/|ref| %.3g, max err/bound %.3g"
           % (name, (np.abs(og - ref) / np.maximum(np.abs(ref), 1e-30)).max(), excess.max()))
    assert excess.max() <= 1.0, excess.max()
