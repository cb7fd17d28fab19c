"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the gated delta rule.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product library (``linear_attention_sequence_rule_amd``) never imports, links
or executes anything here, and nothing here imports the product library: the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, token by token; see its
header for the passages of the pages it follows).  This module only marshals numpy arrays into
that library and builds it with gcc when it is missing.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py`` (closed forms,
special cases, brute-force products, numpy.convolve for the conv prologue).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.gdn_oracle_forward.restype = ctypes.c_int
        lib.gdn_oracle_forward.argtypes = [P] * 13 + [ctypes.c_int] * 5 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_step.restype = ctypes.c_int
        lib.gdn_oracle_step.argtypes = [P] * 9 + [ctypes.c_int] * 5 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_gated_norm.restype = None
        lib.gdn_oracle_gated_norm.argtypes = [P] * 4 + [ctypes.c_long, ctypes.c_int, ctypes.c_double]
        lib.gdn_oracle_gates.restype = None
        lib.gdn_oracle_gates.argtypes = [P] * 6 + [ctypes.c_long, ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, g, beta, initial_state=None, cu_seqlens=None, conv_w=None, *, N=None,
            scale=1.0, l2norm=True, pairs=None, nthreads=0, want_o=True, conv_hist=None, want_conv_hist=False):
    """Token-by-token fp64 gated delta rule over packed sequences.

    q, k: [T_tot, Hk, dk]; v: [T_tot, H, dv]; g, beta: [T_tot, H]; initial_state [N, H, dv, dk]
    or None (zeros); cu_seqlens [N+1] or None (then N equal sequences); conv_w [C, 4] or None
    with C = 2*Hk*dk + H*dv; conv_hist [N, 3, C] or None (zeros): the raw inputs before each
    sequence.  H must be a multiple of Hk; value head h reads query/key head h // (H // Hk).
    ``pairs``: optional iterable of (n, h) to compute; other pairs are left as NaN.
    Returns (o [T_tot, H, dv] or None, final_state [N, H, dv, dk], threads_used), plus the conv
    history after each sequence [N, 3, H*(2dk+dv)] when ``want_conv_hist``.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T_tot, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and H % Hk == 0
    C = 2 * Hk * dk + H * dv
    if cu_seqlens is None:
        if N is None:
            N = 1
        assert T_tot % N == 0
        cu = np.arange(N + 1, dtype=np.int64) * (T_tot // N)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T_tot and np.all(np.diff(cu) >= 0)
    s0 = _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (N, H, dv, dk)
    cw = _f64(conv_w)
    if cw is not None:
        assert cw.shape == (C, 4)
    mask = None
    if pairs is not None:
        mask = np.zeros(N * H, dtype=np.uint8)
        for n, h in pairs:
            mask[n * H + h] = 1
    hist = _f64(conv_hist)
    if hist is not None:
        assert cw is not None and hist.shape == (N, 3, C)
    hout = np.full((N, 3, C), np.nan) if (want_conv_hist and cw is not None) else None
    o = np.full((T_tot, H, dv), np.nan) if want_o else None
    sfin = np.full((N, H, dv, dk), np.nan)
    used = _load().gdn_oracle_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(cu), _ptr(cw), _ptr(hist), _ptr(hout),
        _ptr(o), _ptr(sfin), _ptr(mask), N, H, Hk, dk, dv, float(scale), 1 if l2norm else 0, int(nthreads))
    if want_conv_hist:
        return o, sfin, used, hout
    return o, sfin, used


def step(q, k, v, g, beta, state, *, scale=1.0, l2norm=True, nthreads=0, conv_w=None, conv_hist=None):
    """One decode token per (sequence, head).  q, k [N,Hk,dk]; v [N,H,dv]; g, beta [N,H];
    state [N,H,dv,dk]; optional conv_w [C,4] with conv_hist [N,3,C], C = 2*Hk*dk + H*dv (the three
    previous raw inputs).  Returns (o [N,H,dv], new_state), plus the new conv history when conv_w
    is given, without modifying the inputs."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    N, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and H % Hk == 0
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    assert st.shape == (N, H, dv, dk)
    cw = _f64(conv_w)
    hist = None
    if cw is not None:
        hist = np.array(conv_hist, dtype=np.float64, copy=True, order="C")
        assert hist.shape == (N, 3, 2 * Hk * dk + H * dv)
    o = np.empty((N, H, dv))
    _load().gdn_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cw), _ptr(hist), _ptr(st), _ptr(o),
                            N, H, Hk, dk, dv, float(scale), 1 if l2norm else 0, int(nthreads))
    if cw is not None:
        return o, st, hist
    return o, st


def gates(a, b, A_log, dt_bias):
    """g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b) in fp64.
    a, b [T, H]; A_log, dt_bias [H].  Returns (g, beta) [T, H]."""
    a, b, A_log, dt_bias = (_f64(x) for x in (a, b, A_log, dt_bias))
    T, H = a.shape
    g = np.empty((T, H))
    beta = np.empty((T, H))
    _load().gdn_oracle_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta),
                             T, H)
    return g, beta


def gated_norm(o, z, w, eps):
    """Output epilogue in fp64: each row of o (last axis dv) divided by sqrt(mean(o^2) + eps), times
    (1 + w) and sigmoid(z).  o, z [..., dv]; w [dv].  Returns a new array of o's shape."""
    o, z, w = (_f64(x) for x in (o, z, w))
    assert z.shape == o.shape and w.shape == (o.shape[-1],)
    dv = o.shape[-1]
    out = np.empty_like(o)
    _load().gdn_oracle_gated_norm(_ptr(o), _ptr(z), _ptr(w), _ptr(out), o.size // dv if dv else 0, dv, float(eps))
    return out
