"""Parity with the q/k L2 normalisation switched off (flags without GDN_QK_L2NORM): the kernels take
the norms as 1 and, since the decay bound on a chunk's transition assumes unit keys, never mark a
segment negligible nor stop a transition or rerun early, so the segmented path runs every pass over
whole segments.  q and k are unit rows scaled by 0.9 on the host (then rounded to the storage
type), which keeps the recurrence contracting as the rule assumes; the oracle takes the same
stored values with its normalisation off.  Tolerances as in gdn_testlib.
"""
import numpy as np
import pytest

import gdn_testlib as TL
import oracle
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _unit_rows(wl, name, c=0.9):
    x = wl.as_float(name).astype(np.float64)
    x = c * x / np.linalg.norm(x, axis=-1, keepdims=True)
    x = x.astype(np.float32)
    setattr(wl, name, W.f32_to_bf16_bits(x) if wl.dtype == "bf16" else x)


def _prepare(wl):
    _unit_rows(wl, "q")
    _unit_rows(wl, "k")
    return wl


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 32), ("f32", 32, 64)])
def test_prefill_no_l2norm(dtype, dk, dv):
    wl = _prepare(W.make("nonorm", seed=700 + dk + dv, lengths=[300, 0, 64, 1, 129], H=3, dk=dk, dv=dv,
                         dtype=dtype, s0_std=0.05, varlen=True))
    o, s = TL.run_gpu(wl, l2norm=False)
    o_ref, s_ref = TL.run_oracle(wl, l2norm=False)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("no l2norm %s %d %d %s" % (dtype, dk, dv, e))


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64)])
def test_prefill_no_l2norm_segments(dk, dv):
    """Forced segments without the norm: every transition, entering-state chain and rerun runs in full."""
    wl = _prepare(W.make("nonorm_seg", seed=710 + dv, N=1, T=1000, H=2, dk=dk, dv=dv, dtype="bf16", s0_std=0.02))
    o, s = TL.run_gpu(wl, l2norm=False, segments=3)
    o_ref, s_ref = TL.run_oracle(wl, l2norm=False)
    e = TL.compare(wl, o, s, o_ref, s_ref)
    _flush("no l2norm segments %d %d %s" % (dk, dv, e))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_no_l2norm(dtype):
    from linear_attention_sequence_rule_amd import gdn_recurrent_step
    import torch
    dw = W.decode(N=6, H=3, dk=128, dv=128, dtype=dtype, seed=720, state_std=0.3)
    _unit_rows(dw, "q")
    _unit_rows(dw, "k")
    st = TL.to_dev(dw.state)
    o = gdn_recurrent_step(TL.to_dev(dw.q), TL.to_dev(dw.k), TL.to_dev(dw.v), TL.to_dev(dw.g), TL.to_dev(dw.beta), st,
                           l2norm=False)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.step(dw.as_float("q"), dw.as_float("k"), dw.as_float("v"), dw.g, dw.beta, dw.state,
                               l2norm=False)
    og, sg = TL.o_to_f64(o), st.cpu().numpy().astype(np.float64)
    if dtype == "f32":
        assert np.abs(og - o_ref).max() / np.abs(o_ref).max() <= TL.F32_REL
        assert np.abs(sg - s_ref).max() / np.abs(s_ref).max() <= TL.F32_REL
    else:
        assert np.abs(og - o_ref).max() <= TL.BF16_O_ABS
        d = np.linalg.norm((sg - s_ref).reshape(dw.N * dw.H, -1), axis=1)
        r = np.linalg.norm(s_ref.reshape(dw.N * dw.H, -1), axis=1)
        assert (d / r).max() <= TL.BF16_S_RELF
    _flush("decode no l2norm %s o_abs %.3g" % (dtype, float(np.abs(og - o_ref).max())))
