"""Shared test plumbing: move seeded workloads to the device, run the HIP path through the C ABI
binding, run the fp64 oracle on the same inputs, and compare at the stated tolerances.

Tolerances (the gated delta rule parity bar):
  * fp32 path:  max|gpu - ref| / max|ref| <= 1e-4, on o and on the final state;
  * bf16 path:  o max abs error <= 2e-2; final-state relative Frobenius error <= 1e-2, per
    (sequence, head) and over the whole tensor.
"""
from __future__ import annotations

import numpy as np

import oracle
from linear_attention_sequence_rule_amd import workloads as W

F32_REL = 1e-4
BF16_O_ABS = 2e-2
BF16_S_RELF = 1e-2


def to_dev(x, dtype_tag=None):
    import torch
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def o_to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(wl: W.Workload, *, scale=1.0, l2norm=True, pass_state=True, want_final=True, stream=None, segments=0,
            conv_fused=False):
    from linear_attention_sequence_rule_amd import gdn_chunk_fwd
    import torch
    q, k, v = to_dev(wl.q), to_dev(wl.k), to_dev(wl.v)
    g, beta = to_dev(wl.g), to_dev(wl.beta)
    s0 = to_dev(wl.s0) if pass_state else None
    cu = to_dev(wl.cu_seqlens)
    cw = to_dev(wl.conv_w)
    o, sf = gdn_chunk_fwd(q, k, v, g, beta, s0, cu, cw, N=wl.N, scale=scale, l2norm=l2norm,
                          output_final_state=want_final, stream=stream, segments=segments, conv_fused=conv_fused)
    torch.cuda.synchronize()
    return o_to_f64(o), (sf.cpu().numpy().astype(np.float64) if sf is not None else None)


def run_oracle(wl: W.Workload, *, scale=1.0, l2norm=True, pairs=None, pass_state=True, nthreads=0):
    cu = wl.cu_seqlens
    if cu is None:
        cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    o, sf, _ = oracle.forward(wl.as_float("q"), wl.as_float("k"), wl.as_float("v"), wl.g, wl.beta,
                              wl.s0 if pass_state else None, cu, wl.conv_w, scale=scale,
                              l2norm=l2norm, pairs=pairs, nthreads=nthreads)
    return o, sf


def head_slice(wl: W.Workload, heads) -> W.Workload:
    """The same workload restricted to the given heads (heads are independent chains, so the
    oracle on the slice is exactly the oracle on those heads of the whole workload)."""
    import copy
    hs = np.asarray(list(heads))
    sub = copy.copy(wl)
    sub.H = len(hs)
    sub.q, sub.k, sub.v = (np.ascontiguousarray(x[:, hs]) for x in (wl.q, wl.k, wl.v))
    sub.g, sub.beta = np.ascontiguousarray(wl.g[:, hs]), np.ascontiguousarray(wl.beta[:, hs])
    sub.s0 = None if wl.s0 is None else np.ascontiguousarray(wl.s0[:, hs])
    if wl.conv_w is not None:
        H, dk, dv = wl.H, wl.dk, wl.dv
        rows = np.concatenate([np.arange(h * dk, (h + 1) * dk) for h in hs] +
                              [H * dk + np.arange(h * dk, (h + 1) * dk) for h in hs] +
                              [2 * H * dk + np.arange(h * dv, (h + 1) * dv) for h in hs])
        sub.conv_w = np.ascontiguousarray(wl.conv_w[rows])
    return sub


def pair_rows(wl, n, h):
    cu = np.concatenate([[0], np.cumsum(wl.lengths)])
    return slice(int(cu[n]), int(cu[n + 1])), h


def compare(wl, o_gpu, s_gpu, o_ref, s_ref, pairs=None, f32=None):
    """Assert parity; returns a dict of the measured errors."""
    f32 = (wl.dtype == "f32") if f32 is None else f32
    if pairs is None:
        pairs = wl.pairs()
    errs = {"o_abs": 0.0, "o_ref_max": 0.0, "s_relF_worst": 0.0, "s_abs": 0.0, "s_ref_max": 0.0,
            "o_worst_pair": None, "s_worst_pair": None}
    s_num = s_den = 0.0
    for n, h in pairs:
        rows, hh = pair_rows(wl, n, h)
        a, b = o_gpu[rows, hh], o_ref[rows, hh]
        assert np.all(np.isfinite(a)), "non-finite o at pair %s" % ((n, h),)
        if a.size:
            oe = float(np.abs(a - b).max())
            if errs["o_worst_pair"] is None or oe > errs["o_abs"]:
                errs["o_worst_pair"] = (int(n), int(h))
            errs["o_abs"] = max(errs["o_abs"], oe)
            errs["o_ref_max"] = max(errs["o_ref_max"], float(np.abs(b).max()))
        if s_gpu is not None:
            sa, sb = s_gpu[n, h], s_ref[n, h]
            assert np.all(np.isfinite(sa)), "non-finite state at pair %s" % ((n, h),)
            d = float(np.linalg.norm(sa - sb))
            r = float(np.linalg.norm(sb))
            s_num += d * d
            s_den += r * r
            if errs["s_worst_pair"] is None or d / max(r, 1e-30) > errs["s_relF_worst"]:
                errs["s_worst_pair"] = (int(n), int(h))
            errs["s_relF_worst"] = max(errs["s_relF_worst"], d / max(r, 1e-30))
            errs["s_abs"] = max(errs["s_abs"], float(np.abs(sa - sb).max()))
            errs["s_ref_max"] = max(errs["s_ref_max"], float(np.abs(sb).max()))
    errs["s_relF_all"] = (s_num ** 0.5) / max(s_den ** 0.5, 1e-30)
    if f32:
        o_rel = errs["o_abs"] / max(errs["o_ref_max"], 1e-30)
        errs["o_rel"] = o_rel
        assert o_rel <= F32_REL, errs
        if s_gpu is not None:
            s_rel = errs["s_abs"] / max(errs["s_ref_max"], 1e-30)
            errs["s_rel"] = s_rel
            assert s_rel <= F32_REL, errs
    else:
        assert errs["o_abs"] <= BF16_O_ABS, errs
        if s_gpu is not None:
            assert errs["s_relF_worst"] <= BF16_S_RELF, errs
            assert errs["s_relF_all"] <= BF16_S_RELF, errs
    return errs
