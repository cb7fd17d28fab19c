"""Parity of the HIP path (through the C ABI) against the fp64 oracle on identical seeded inputs.

Sizes span several 64-token chunks and ragged tails; the named workloads run at full size (the long
prefill and the varlen workload, every chain of each, in test_gpu_full_workloads.py).
"""
import numpy as np
import pytest

import gdn_testlib as TL
import oracle
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------------- prefill

def test_tiny_f32_workload():
    """B=1, T=256, H=2, d=32, fp32, zero initial state, seed 0: max relative error <= 1e-4."""
    wl = W.tiny_f32()
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("tiny_f32 %s" % e)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
def test_f32_ragged_varlen(dk, dv):
    wl = W.make("f32_ragged", seed=100 + dk + dv, lengths=[130, 0, 64, 1, 77], H=3, dk=dk, dv=dv,
                dtype="f32", s0_std=0.5, varlen=True)
    o, s = TL.run_gpu(wl, scale=0.5)
    o_ref, s_ref = TL.run_oracle(wl, scale=0.5)
    TL.compare(wl, o, s, o_ref, s_ref)
    # zero-length sequence: final state equals the initial one exactly
    np.testing.assert_array_equal(s[1], wl.s0[1])


def test_f32_equal_lengths_no_state():
    wl = W.make("f32_eq", seed=7, N=3, T=190, H=2, dk=64, dv=64, dtype="f32")
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    TL.compare(wl, o, s, o_ref, s_ref)


def test_f32_conv_prologue():
    wl = W.make("f32_conv", seed=8, lengths=[70, 3, 129], H=2, dk=32, dv=64, dtype="f32", s0_std=0.1,
                conv=True, varlen=True)
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    TL.compare(wl, o, s, o_ref, s_ref)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32), (32, 64), (128, 32), (64, 128)])
def test_bf16_ragged_varlen(dk, dv):
    wl = W.make("bf16_ragged", seed=200 + dk + dv, lengths=[300, 0, 64, 1, 129], H=4, dk=dk, dv=dv,
                dtype="bf16", s0_std=0.02, varlen=True)
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("bf16_ragged %d %d %s" % (dk, dv, e))
    np.testing.assert_array_equal(s[1], wl.s0[1])


@pytest.mark.parametrize("dk,dv,segs", [(128, 128, 0), (64, 32, 0), (128, 128, 3), (128, 64, 2)])
def test_bf16_output_scale(dk, dv, segs):
    """A negative, non-unit output scale.  The chunk kernels carry it inside the prepared output
    operands (Pm' and the state part's row factors), including the first-chunk operands that the
    first pass keeps for the segment reruns, so the segmented cases cover those too."""
    wl = W.make("bf16_scale", seed=500 + dk + dv + segs, N=2, T=700, H=3, dk=dk, dv=dv, dtype="bf16", s0_std=0.02)
    o, s = TL.run_gpu(wl, scale=-0.37, segments=segs)
    o_ref, s_ref = TL.run_oracle(wl, scale=-0.37)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("bf16 scale -0.37 %d %d segs=%d %s" % (dk, dv, segs, e))


def test_bf16_conv_varlen_small():
    wl = W.varlen(lengths=[520, 64, 7, 1000], H=4)
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("bf16_conv %s" % e)


@pytest.mark.parametrize("dk,dv", [(64, 32), (32, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("fused", [False, True])
def test_bf16_conv_dims(dk, dv, fused):
    """The conv prologue as a separate pass (default for 64/32-row workgroups) and inside the chunk
    kernel (GDN_CONV_FUSED, and always for 128-row workgroups: dk = dv = 128)."""
    wl = W.make("bf16_conv", seed=300 + dk + dv, lengths=[200, 3, 64, 0, 131], H=3, dk=dk, dv=dv, dtype="bf16",
                s0_std=0.05, conv=True, varlen=True)
    o, s = TL.run_gpu(wl, scale=0.8, conv_fused=fused)
    o_ref, s_ref = TL.run_oracle(wl, scale=0.8)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("bf16_conv %d %d fused=%s %s" % (dk, dv, fused, e))


@pytest.mark.parametrize("dv,fused", [(64, False), (64, True), (128, False)])
def test_bf16_conv_segments(dv, fused):
    """Conv prologue on the segmented path: segments that start inside a sequence take the three
    previous raw tokens as conv history; one head decays slowly so the corrections run long.
    dv = 128: 128-row workgroups, conv inside the kernel in every pass."""
    wl = W.make("conv_seg", seed=51 + dv, lengths=[700, 130, 1, 520], H=2, dk=128, dv=dv, dtype="bf16", s0_std=0.02,
                conv=True, varlen=True)
    wl.g[:, 1] = -1e-3
    o, s = TL.run_gpu(wl, segments=3, conv_fused=fused)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("conv segments dv=%d fused=%s %s" % (dv, fused, e))


def test_bf16_slow_decay():
    """Slow decay (g ~ -1e-3) keeps the whole history alive: the hardest case for bf16 operands."""
    wl = W.make("slow", seed=9, N=2, T=1024, H=4, dk=128, dv=128, dtype="bf16", s0_std=0.02)
    wl.g = np.full_like(wl.g, -1e-3)
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("slow_decay %s" % e)


def test_prefill_workload_full():
    """B=4, T=4096, H=16, d=128, bf16, initial state ~N(0, 0.02): every chain checked."""
    wl = W.prefill()
    o, s = TL.run_gpu(wl)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("prefill full %s" % e)


# ------------------------------------------------------------------- segmented long sequences

@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("segs", [2, 3, 5])
def test_bf16_segments_forced(segs, dv):
    """Sequences cut into segments (the last one empty for segs=5); workload gates, so transitions
    and corrections stop at the decay bound after a chunk or two.  dv = 64: 64-row workgroups;
    dv = 128: 128-row workgroups in every pass."""
    wl = W.make("seg", seed=40 + segs + dv, N=2, T=1000, H=3, dk=128, dv=dv, dtype="bf16", s0_std=0.02)
    o, s = TL.run_gpu(wl, segments=segs)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("segments %d dv=%d %s" % (segs, dv, e))


def test_bf16_segments_slow_decay_mixed():
    """Head 0 decays slowly (g = -1e-3: full transitions A_p, full reruns, chained entering states);
    heads 1, 2 keep the workload gates (negligible transitions).  No initial state passed."""
    wl = W.make("seg_slow", seed=47, N=1, T=1024, H=3, dk=128, dv=128, dtype="bf16")
    wl.g[:, 0] = -1e-3
    o, s = TL.run_gpu(wl, segments=4)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("segments slow %s" % e)


@pytest.mark.parametrize("dk", [32, 64, 128])
def test_bf16_segments_queued_slow_decay(dk):
    """d_k = d_v: the transition and rerun passes share one launch.  3 sequences x 8 segments x 16
    heads = 384 workgroups, more than the 256 compute units hold at once (one per unit at every
    width), and every third head decays slowly (g = -1e-3), so its transitions are formed in full
    and the reruns of later segments wait for them, some of them for workgroups that start only
    after others have begun to wait."""
    wl = W.make("seg_queue", seed=50 + dk, N=3, T=1024, H=16, dk=dk, dv=dk, dtype="bf16", s0_std=0.02)
    wl.g[:, ::3] = -1e-3
    o, s = TL.run_gpu(wl, segments=8)
    o_ref, s_ref = TL.run_oracle(wl)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("segments queued slow dk=dv=%d %s" % (dk, e))


@pytest.mark.parametrize("dk,dv", [(64, 128), (32, 32), (128, 128)])
def test_bf16_segments_varlen(dk, dv):
    wl = W.make("seg_var", seed=48 + dk, lengths=[300, 0, 64, 1, 700], H=2, dk=dk, dv=dv, dtype="bf16",
                s0_std=0.05, varlen=True)
    wl.g[:, 1] = -2e-3
    o, s = TL.run_gpu(wl, segments=3)
    o_ref, s_ref = TL.run_oracle(wl)
    TL.compare(wl, o, s, o_ref, s_ref)
    np.testing.assert_array_equal(s[1], wl.s0[1])


def test_bf16_segments_without_final_state():
    wl = W.make("seg_nofinal", seed=49, N=1, T=700, H=2, dk=64, dv=64, dtype="bf16", s0_std=0.02)
    o, s = TL.run_gpu(wl, segments=3, want_final=False)
    assert s is None
    o_ref, _ = TL.run_oracle(wl)
    TL.compare(wl, o, None, o_ref, None)


# ----------------------------------------------------------------------------------- decode

def _decode_check(dw, scale=1.0):
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    st = TL.to_dev(dw.state)
    o = gdn_recurrent_step(TL.to_dev(dw.q), TL.to_dev(dw.k), TL.to_dev(dw.v), TL.to_dev(dw.g), TL.to_dev(dw.beta), st,
                           scale=scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state,
                               scale=scale)
    og = TL.o_to_f64(o)
    sg = st.cpu().numpy().astype(np.float64)
    if dw.dtype == "f32":
        assert np.abs(og - o_ref).max() / np.abs(o_ref).max() <= TL.F32_REL
        assert np.abs(sg - s_ref).max() / np.abs(s_ref).max() <= TL.F32_REL
    else:
        assert np.abs(og - o_ref).max() <= TL.BF16_O_ABS
        d = np.linalg.norm((sg - s_ref).reshape(dw.N * dw.H, -1), axis=1)
        r = np.linalg.norm(s_ref.reshape(dw.N * dw.H, -1), axis=1)
        assert (d / r).max() <= TL.BF16_S_RELF
    return float(np.abs(og - o_ref).max())


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (64, 64), (128, 32), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_dims(dk, dv, dtype):
    dw = W.decode(N=5, H=3, dk=dk, dv=dv, dtype=dtype, seed=dk * 3 + dv, state_std=0.3)
    _decode_check(dw, scale=0.75)


def test_decode_workload_full():
    """256 sequences x 32 heads, d=128, bf16 tokens, fp32 state ~N(0, 0.02) (512 MiB), in place."""
    dw = W.decode()
    err = _decode_check(dw)
    _flush("decode full o_abs=%g" % err)


def test_decode_then_prefill_consistency():
    """prefill(T) followed by one decode step equals prefill(T+1) (within bf16 tolerance)."""
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    wl = W.make("pd", seed=31, N=2, T=129, H=2, dk=128, dv=128, dtype="bf16", s0_std=0.02)
    q, k, v = TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v)
    g, b = TL.to_dev(wl.g), TL.to_dev(wl.beta)
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    o_full, s_full = gdn_chunk_fwd(q, k, v, g, b, TL.to_dev(wl.s0), N=2)
    # first 128 tokens of each sequence, then one step
    idx = torch.cat([torch.arange(0, 128), torch.arange(129, 257)]).cuda()
    last = torch.tensor([128, 257]).cuda()
    o_a, s_a = gdn_chunk_fwd(q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous(), g[idx].contiguous(),
                             b[idx].contiguous(), TL.to_dev(wl.s0), N=2)
    o_step = gdn_recurrent_step(q[last].contiguous(), k[last].contiguous(), v[last].contiguous(),
                                g[last].contiguous(), b[last].contiguous(), s_a)
    torch.cuda.synchronize()
    assert (o_step.float() - o_full[last].float()).abs().max().item() <= TL.BF16_O_ABS
    rel = ((s_a - s_full).norm() / s_full.norm()).item()
    assert rel <= TL.BF16_S_RELF


def test_side_stream_and_no_final_state():
    """Both calls on a caller-provided stream (created at the default priority, waiting for the
    uploads on the current stream); the 128-row segmented path without a final state."""
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd, gdn_recurrent_step
    import torch
    wl = W.make("side", seed=91, lengths=[700, 65, 3], H=2, dk=128, dv=128, dtype="bf16", s0_std=0.02, varlen=True)
    q, k, v = TL.to_dev(wl.q), TL.to_dev(wl.k), TL.to_dev(wl.v)
    g, beta, s0, cu = TL.to_dev(wl.g), TL.to_dev(wl.beta), TL.to_dev(wl.s0), TL.to_dev(wl.cu_seqlens)
    dw = W.decode(N=4, H=2, seed=92)
    dq, dk_, dv_, dg, db, st = (TL.to_dev(x) for x in (dw.q, dw.k, dw.v, dw.g, dw.beta, dw.state))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o, sf = gdn_chunk_fwd(q, k, v, g, beta, s0, cu, N=wl.N, segments=2, output_final_state=False, stream=side)
        od = gdn_recurrent_step(dq, dk_, dv_, dg, db, st, stream=side)
    side.synchronize()
    assert sf is None
    o_ref, _ = TL.run_oracle(wl)
    TL.compare(wl, TL.o_to_f64(o), None, o_ref, None)
    od_ref, st_ref = oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state)
    assert np.abs(TL.o_to_f64(od) - od_ref).max() <= TL.BF16_O_ABS
    d = np.linalg.norm((st.cpu().numpy().astype(np.float64) - st_ref).reshape(dw.N * dw.H, -1), axis=1)
    assert (d / np.linalg.norm(st_ref.reshape(dw.N * dw.H, -1), axis=1)).max() <= TL.BF16_S_RELF
