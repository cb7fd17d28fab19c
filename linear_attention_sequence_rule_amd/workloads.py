"""Seeded synthetic workloads for the gated delta rule (inputs only).

This module draws the inputs that both the HIP path and the CPU oracle consume.  It holds none
of the rule's arithmetic: it draws random numbers, applies the configs' stated input recipe for
the gates (g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b): the distribution of the
g and beta inputs, as the gate parameterisation on page maplevalley.com.cn/news/1910399,
section 2.1 gives it) and rounds to the storage dtype.

Recipe (every draw comes from its own numpy PCG64 stream, keyed by
``(seed, tensor id, sequence, token block)``, so blocks can be drawn in parallel and any one
(sequence, head) can be re-drawn alone):

* q, k, v ~ N(0, 1) drawn as float32, rounded to bf16 with round-to-nearest-even for the bf16
  workloads (kept fp32 for the fp32 one).  q and k are L2-normalised inside the kernels.
* A_log ~ U(0, ln 16) [H], dt_bias ~ N(0, 0.5) [H], a ~ N(0, 1) [T, H], b ~ N(0, 1) [T, H];
  g and beta are evaluated in float64 and rounded to float32.
* initial states ~ N(0, 0.02) fp32 where the workload has them.
* varlen lengths ~ U{512..16384} (inclusive integers); conv weights ~ N(0, 0.5) fp32.

The five named workloads are the prefill/decode shapes of the gated-delta-rule benchmark
suite: ``tiny_f32`` (B=1, T=256, H=2, d=32), ``prefill`` (B=4, T=4096, H=16, d=128),
``long_prefill`` (B=1, T=262144, H=16, d=128), ``decode`` (256 sequences x 32 heads, d=128)
and ``varlen`` (64 sequences of 512..16384 tokens, H=32, d=128, conv prologue).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

TOKEN_BLOCK = 4096
_IDS = {"lengths": 0, "A_log": 1, "dt_bias": 2, "a": 3, "b": 4, "q": 5, "k": 6, "v": 7,
        "s0": 8, "conv_w": 9, "conv_hist": 10}


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed, name, *idx):
    return np.random.default_rng([int(seed), _IDS[name], *[int(i) for i in idx]])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """Inputs of one gdn_chunk_fwd / gdn_recurrent_step call, host side.

    q, k, v are uint16 bf16 bit patterns (dtype 'bf16') or float32 (dtype 'f32').  H counts the
    value heads; q and k have Hk query/key heads (``q.shape[1]``), Hk = H unless grouped.
    """
    name: str
    dtype: str
    N: int
    H: int
    dk: int
    dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    s0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    conv_w: Optional[np.ndarray]
    lengths: np.ndarray
    chunk: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def T_tot(self) -> int:
        return int(self.q.shape[0])

    @property
    def Hk(self) -> int:
        return int(self.q.shape[1])

    def as_float(self, name: str) -> np.ndarray:
        """q/k/v (or any array field) widened exactly to float32."""
        x = getattr(self, name)
        if x is None:
            return None
        if x.dtype == np.uint16:
            return bf16_bits_to_f32(x)
        return x

    def pairs(self):
        return [(n, h) for n in range(self.N) for h in range(self.H)]


def _normal_tokens(seed, name, lengths, H, d, dtype, pool):
    """[sum(lengths), H, d] standard normals, drawn per (sequence, token block)."""
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    out = np.empty((T, H, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    jobs = []
    for n, L in enumerate(lengths):
        for blk in range(0, int(L), TOKEN_BLOCK):
            jobs.append((n, blk, min(TOKEN_BLOCK, int(L) - blk)))

    def fill(job):
        n, blk, cnt = job
        x = _rng(seed, name, n, blk // TOKEN_BLOCK).standard_normal((cnt, H, d), dtype=np.float32)
        s = offs[n] + blk
        out[s:s + cnt] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    list(pool.map(fill, jobs))
    return out


def _gates(seed, lengths, H):
    """g, beta [T, H] float32 from the configs' recipe, drawn per sequence."""
    A_log = _rng(seed, "A_log").uniform(0.0, math.log(16.0), size=H)
    dt_bias = _rng(seed, "dt_bias").normal(0.0, 0.5, size=H)
    gs, bs = [], []
    for n, L in enumerate(lengths):
        a = _rng(seed, "a", n).standard_normal((int(L), H))
        b = _rng(seed, "b", n).standard_normal((int(L), H))
        x = a + dt_bias[None, :]
        softplus = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
        gs.append((-np.exp(A_log)[None, :] * softplus).astype(np.float32))
        bs.append((1.0 / (1.0 + np.exp(-b))).astype(np.float32))
    g = np.concatenate(gs) if gs else np.zeros((0, H), np.float32)
    beta = np.concatenate(bs) if bs else np.zeros((0, H), np.float32)
    return np.ascontiguousarray(g), np.ascontiguousarray(beta), A_log, dt_bias


def raw_gates(seed, lengths, H):
    """The raw gate draws (a, b [T,H]; A_log, dt_bias [H]) behind ``_gates``, float64."""
    A_log = _rng(seed, "A_log").uniform(0.0, math.log(16.0), size=H)
    dt_bias = _rng(seed, "dt_bias").normal(0.0, 0.5, size=H)
    a = np.concatenate([_rng(seed, "a", n).standard_normal((int(L), H))
                        for n, L in enumerate(lengths)])
    b = np.concatenate([_rng(seed, "b", n).standard_normal((int(L), H))
                        for n, L in enumerate(lengths)])
    return a, b, A_log, dt_bias


def raw_gate_inputs(seed, lengths, H):
    """The raw gate inputs as a caller passes them with gate_params: a, b [T, H] float32 and
    gate_params [2, H] float32 (row 0 = A_log, row 1 = dt_bias), from the draws of ``raw_gates``."""
    a, b, A_log, dt_bias = raw_gates(seed, lengths, H)
    gp = np.stack([A_log, dt_bias]).astype(np.float32)
    return a.astype(np.float32), b.astype(np.float32), np.ascontiguousarray(gp)


def conv_inputs(seed, N, H, dk, dv, dtype, Hk=None):
    """Conv weights ~N(0, 0.5) [C, 4] float32 and a conv history [N, 3, C] of standard normals in
    the storage dtype (bf16 bit patterns or float32): the three raw inputs before each sequence, as
    a previous call would have left them.  C = 2 Hk dk + H dv conv channels (Hk = H by default)."""
    Hk = H if Hk is None else Hk
    C = 2 * Hk * dk + H * dv
    cw = _rng(seed, "conv_w").normal(0.0, 0.5, size=(C, 4)).astype(np.float32)
    x = _rng(seed, "conv_hist").standard_normal((N, 3, C), dtype=np.float32)
    return cw, (f32_to_bf16_bits(x) if dtype == "bf16" else x)


def _states(seed, N, H, dv, dk, std, pool):
    out = np.empty((N, H, dv, dk), dtype=np.float32)

    def fill(n):
        out[n] = _rng(seed, "s0", n).normal(0.0, std, size=(H, dv, dk)).astype(np.float32)

    list(pool.map(fill, range(N)))
    return out


def make(name="custom", *, seed=0, N=1, T=None, lengths=None, H=2, dk=32, dv=32, dtype="bf16",
         s0_std=None, conv=False, varlen=False, chunk=64, Hk=None) -> Workload:
    """Draw one prefill workload.

    ``lengths`` (list) gives per-sequence token counts; otherwise N sequences of T tokens.
    ``Hk`` query/key heads shared by groups of the H value heads (default: Hk = H).
    ``varlen`` marks the workload as packed (cu_seqlens passed to the kernels even when the
    lengths happen to be equal).  ``s0_std`` None means a zero initial state (passed as NULL).
    """
    if lengths is None:
        lengths = [int(T)] * N
    lengths = np.asarray(lengths, dtype=np.int64)
    N = len(lengths)
    with ThreadPoolExecutor(_workers()) as pool:
        Hk = H if Hk is None else Hk
        q = _normal_tokens(seed, "q", lengths, Hk, dk, dtype, pool)
        k = _normal_tokens(seed, "k", lengths, Hk, dk, dtype, pool)
        v = _normal_tokens(seed, "v", lengths, H, dv, dtype, pool)
        g, beta, A_log, dt_bias = _gates(seed, lengths, H)
        s0 = _states(seed, N, H, dv, dk, s0_std, pool) if s0_std is not None else None
    cw = None
    if conv:
        cw = _rng(seed, "conv_w").normal(0.0, 0.5, size=(2 * Hk * dk + H * dv, 4)).astype(np.float32)
    cu = None
    if varlen:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return Workload(name=name, dtype=dtype, N=N, H=H, dk=dk, dv=dv, q=q, k=k, v=v, g=g,
                    beta=beta, s0=s0, cu_seqlens=cu, conv_w=cw, lengths=lengths, chunk=chunk,
                    meta={"seed": seed, "A_log": A_log, "dt_bias": dt_bias})


def varlen_lengths(seed, n_seq=64, lo=512, hi=16384):
    return _rng(seed, "lengths").integers(lo, hi + 1, size=n_seq)


# --- the named workloads -------------------------------------------------------------------

def tiny_f32(**kw):
    """B=1, T=256, H=2, d_k=d_v=32, fp32, chunk 64, zero initial state, seed 0."""
    args = dict(name="tiny_f32", seed=0, N=1, T=256, H=2, dk=32, dv=32, dtype="f32")
    args.update(kw)
    return make(**args)


def prefill(**kw):
    """B=4, T=4096, H=16, d=128, bf16 q/k/v, initial state ~N(0, 0.02), seed 1."""
    args = dict(name="prefill", seed=1, N=4, T=4096, H=16, dk=128, dv=128, dtype="bf16",
                s0_std=0.02)
    args.update(kw)
    return make(**args)


def long_prefill(**kw):
    """B=1, T=262144, H=16, d=128, bf16, zero initial state, seed 2."""
    args = dict(name="long_prefill", seed=2, N=1, T=262144, H=16, dk=128, dv=128, dtype="bf16")
    args.update(kw)
    return make(**args)


def varlen(n_seq=64, lo=512, hi=16384, **kw):
    """64 sequences, lengths ~U{512..16384}, packed via cu_seqlens, H=32, d=128, bf16, conv
    (4 taps, weights ~N(0, 0.5)) + SiLU prologue, initial states ~N(0, 0.02), seed 4."""
    seed = kw.pop("seed", 4)
    lengths = kw.pop("lengths", None)
    if lengths is None:
        lengths = varlen_lengths(seed, n_seq, lo, hi)
    args = dict(name="varlen", seed=seed, lengths=lengths, H=32, dk=128, dv=128, dtype="bf16",
                s0_std=0.02, conv=True, varlen=True)
    args.update(kw)
    return make(**args)


@dataclass
class DecodeWorkload:
    name: str
    dtype: str
    N: int
    H: int
    dk: int
    dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state: np.ndarray

    def as_float(self, name: str) -> np.ndarray:
        x = getattr(self, name)
        return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x

    @property
    def Hk(self) -> int:
        return int(self.q.shape[1])


def decode(N=256, H=32, dk=128, dv=128, dtype="bf16", seed=3, state_std=0.02, name="decode", Hk=None):
    """One token per sequence: 256 sequences x 32 heads, d=128, bf16 q/k/v, fp32 state
    ~N(0, 0.02) (512 MiB), gates as for prefill, seed 3."""
    lengths = np.ones(N, dtype=np.int64)
    with ThreadPoolExecutor(_workers()) as pool:
        Hk = H if Hk is None else Hk
        q = _normal_tokens(seed, "q", lengths, Hk, dk, dtype, pool)
        k = _normal_tokens(seed, "k", lengths, Hk, dk, dtype, pool)
        v = _normal_tokens(seed, "v", lengths, H, dv, dtype, pool)
        g, beta, _, _ = _gates(seed, lengths, H)
        st = _states(seed, N, H, dv, dk, state_std, pool)
    return DecodeWorkload(name=name, dtype=dtype, N=N, H=H, dk=dk, dv=dv, q=q, k=k, v=v, g=g,
                          beta=beta, state=st)
