"""The Python binding rejects mis-shaped tensors before anything reaches the library.

The C ABI takes raw device pointers and cannot see buffer sizes, so a short o, final_state, g or
state would be written or read out of bounds on the device.  The binding checks every tensor's shape
against the header's ([T_tot, H] gates, [N, H, dv, dk] states, [C, 4] conv weights with
C = 2 Hk dk + H dv, ...) first, so these tests need neither a GPU nor the library: host tensors of
the wrong shape raise ValueError naming the shape, and a well-shaped host tensor passes the shape
checks and fails only at the device-placement check that follows.
"""
import pytest
import torch

import linear_attention_sequence_rule_amd as gdn

T, H, HK, DK, DV, N = 10, 4, 2, 32, 64, 2
CC = 2 * HK * DK + H * DV


def _prefill_args():
    f = torch.float32
    return dict(q=torch.zeros(T, HK, DK), k=torch.zeros(T, HK, DK), v=torch.zeros(T, H, DV),
                g=torch.zeros(T, H), beta=torch.zeros(T, H), initial_state=torch.zeros(N, H, DV, DK, dtype=f),
                cu_seqlens=torch.tensor([0, 4, T], dtype=torch.int32))


def _call_prefill(**over):
    a = _prefill_args()
    kw = {}
    for name in ("conv_w", "conv_state", "out_gate", "norm_weight", "o", "final_state", "gate_params"):
        if name in over:
            kw[name] = over.pop(name)
    a.update(over)
    return gdn.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"], a["cu_seqlens"],
                             kw.pop("conv_w", None), **kw)


BAD_PREFILL = {
    "k": torch.zeros(T, HK, DK + 1),
    "v": torch.zeros(T - 1, H, DV),
    "g": torch.zeros(T, H - 1),
    "beta": torch.zeros(T + 1, H),
    "initial_state": torch.zeros(N, H, DK, DV),
    "final_state": torch.zeros(N + 1, H, DV, DK),
    "o": torch.zeros(T, H, DV // 2),
    "gate_params": torch.zeros(H, 2),
    "conv_w": torch.zeros(CC - 1, 4),
    "out_gate": torch.zeros(T, H, DV - 1),
    "norm_weight": torch.zeros(DV + 1),
}


@pytest.mark.parametrize("name", sorted(BAD_PREFILL))
def test_prefill_rejects_bad_shape(name):
    with pytest.raises(ValueError, match="%s must have shape" % name):
        _call_prefill(**{name: BAD_PREFILL[name]})


def test_prefill_conv_state_shape():
    with pytest.raises(ValueError, match="conv_state must have shape"):
        _call_prefill(conv_w=torch.zeros(CC, 4), conv_state=torch.zeros(N, 4, CC))


def test_prefill_rank():
    with pytest.raises(ValueError, match="q must have 3 dimensions"):
        _call_prefill(q=torch.zeros(T, HK * DK))


def test_prefill_good_shapes_reach_device_check():
    """Correct shapes pass every shape check; the host tensors then fail the placement check."""
    with pytest.raises(ValueError, match="device tensor"):
        _call_prefill(conv_w=torch.zeros(CC, 4), conv_state=torch.zeros(N, 3, CC),
                      out_gate=torch.zeros(T, H, DV), norm_weight=torch.zeros(DV),
                      o=torch.zeros(T, H, DV), final_state=torch.zeros(N, H, DV, DK))


def _step_args():
    return dict(q=torch.zeros(N, HK, DK), k=torch.zeros(N, HK, DK), v=torch.zeros(N, H, DV),
                g=torch.zeros(N, H), beta=torch.zeros(N, H), state=torch.zeros(N, H, DV, DK))


BAD_STEP = {
    "k": torch.zeros(N, HK + 1, DK),
    "v": torch.zeros(N + 1, H, DV),
    "g": torch.zeros(N + 1, H),
    "beta": torch.zeros(N, 1),
    "state": torch.zeros(N, H, DV, DK // 2),
    "o": torch.zeros(N, H - 1, DV),
    "gate_params": torch.zeros(2, H + 1),
    "conv_w": torch.zeros(CC, 3),
    "out_gate": torch.zeros(N, H, 1),
    "norm_weight": torch.zeros(1),
}


@pytest.mark.parametrize("name", sorted(BAD_STEP))
def test_step_rejects_bad_shape(name):
    a = _step_args()
    kw = {}
    if name in a:
        a[name] = BAD_STEP[name]
    else:
        kw[name] = BAD_STEP[name]
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gdn.gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], **kw)


def test_step_good_shapes_reach_device_check():
    a = _step_args()
    with pytest.raises(ValueError, match="device tensor"):
        gdn.gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], o=torch.zeros(N, H, DV),
                               conv_w=torch.zeros(CC, 4), conv_state=torch.zeros(N, 3, CC))
