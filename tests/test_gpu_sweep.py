"""A seeded sweep over combinations of the prefill options, each against the fp64 oracle at the
bars of gdn_testlib: precision (bf16, fp32), head sizes (d_k = d_v, where the segmented path runs
its transition and rerun passes in one launch, and d_k != d_v, where they run as two launches),
value heads sharing query/key heads, packed ragged lengths with empty and one-token sequences,
forced segment counts, slowly decaying heads (transitions formed in full, reruns waiting for
them), the conv prologue in the kernel or as a streaming pass, initial states present or absent,
and a non-unit output scale.  The cases are drawn once from a fixed seed, so every run checks the
same ones; each is small enough for the oracle to finish in well under a second.
"""
import numpy as np
import pytest

import gdn_testlib as TL
from linear_attention_sequence_rule_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(32, 32), (64, 64), (128, 128), (64, 128), (128, 64), (32, 128), (128, 32)]


def _cases(n=28, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dk, dv = SHAPES[i % len(SHAPES)]
        dtype = "f32" if i % 5 == 3 else "bf16"
        H = int(rng.integers(1, 5))
        Hk = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
        nseq = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.choice([0, 1, 17, 64, 65, 200, 333, 640, 1100], size=nseq)]
        if sum(lengths) == 0:
            lengths[0] = 129
        segments = 0 if dtype == "f32" else int(rng.choice([0, 1, 2, 3, 5, 6]))
        slow = [h for h in range(H) if rng.random() < 0.35]
        conv = bool(rng.random() < 0.4)
        conv_fused = bool(conv and dtype == "bf16" and rng.random() < 0.5)
        s0 = bool(rng.random() < 0.7)
        scale = float(rng.choice([1.0, 0.5, -0.37]))
        out.append(dict(i=i, dk=dk, dv=dv, dtype=dtype, H=H, Hk=Hk, lengths=lengths, segments=segments, slow=slow,
                        conv=conv, conv_fused=conv_fused, s0=s0, scale=scale))
    return out


CASES = _cases()


def _id(c):
    return "%d-%s-%dx%d-H%d/%d-L%s-P%d-slow%s%s%s%s" % (
        c["i"], c["dtype"], c["dk"], c["dv"], c["H"], c["Hk"], "_".join(map(str, c["lengths"])), c["segments"],
        "".join(map(str, c["slow"])) or "-", "-conv" if c["conv"] else "", "F" if c["conv_fused"] else "",
        "-s0" if c["s0"] else "")


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_prefill_sweep(c):
    wl = W.make("sweep", seed=900 + c["i"], lengths=c["lengths"], H=c["H"], Hk=c["Hk"], dk=c["dk"], dv=c["dv"],
                dtype=c["dtype"], s0_std=0.03 if c["s0"] else None, conv=c["conv"], varlen=True)
    for h in c["slow"]:
        wl.g[:, h] = -1.5e-3
    print("case %s" % _id(c), flush=True)
    o, s = TL.run_gpu(wl, scale=c["scale"], segments=c["segments"], conv_fused=c["conv_fused"])
    o_ref, s_ref = TL.run_oracle(wl, scale=c["scale"])
    e = TL.compare(wl, o, s, o_ref, s_ref)
    print("  o_abs %.3g  s_relF %.3g" % (e["o_abs"], e["s_relF_worst"]), flush=True)
