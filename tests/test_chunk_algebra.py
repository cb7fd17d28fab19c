"""The chunked form the kernels evaluate, in plain fp64 numpy, against the token-by-token oracle.

The pages say only that the sequence is cut into chunks computed in parallel inside, with the
state carried serially between chunks (page pzsr.cn/news/750, section 1、为什么要设计为chunk的模式);
they give no chunk algebra.  The form below is derived from the rule
S_t = alpha_t S_{t-1} + u_t k_t^T, u_t = beta_t (v_t - alpha_t S_{t-1} k_t):

  gamma_i = sum_{s<=i} g_s (inside the chunk), Gamma_i = exp(gamma_i), M_ij = exp(gamma_i - gamma_j), j<=i
  L  = strict_lower(diag(beta) (M o K K^T)),  T = (I + L)^-1
  U  = T (diag(beta) V - diag(beta Gamma) K S^T)            (the u_t of the chunk, stacked)
  O  = diag(Gamma) Q S^T + lower(M o Q K^T) U
  S' = Gamma_C S + U^T diag(exp(gamma_C - gamma)) K

Every decay factor is exp of a non-positive number, so nothing overflows.
"""
import math

import numpy as np
import pytest

import oracle


def unit_rows(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


def chunked(q, k, v, g, beta, s0, C):
    T = q.shape[0]
    S = s0.copy()
    out = np.zeros_like(v)
    for a in range(0, T, C):
        b = min(a + C, T)
        Q, K, V, gg, bb = q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b]
        n = b - a
        gam = np.cumsum(gg)
        M = np.tril(np.exp(gam[:, None] - gam[None, :]))
        L = np.tril(bb[:, None] * M * (K @ K.T), -1)
        Tm = np.linalg.inv(np.eye(n) + L)
        U = Tm @ (bb[:, None] * V - (bb * np.exp(gam))[:, None] * (K @ S.T))
        out[a:b] = np.exp(gam)[:, None] * (Q @ S.T) + (M * (Q @ K.T)) @ U
        S = math.exp(gam[-1]) * S + U.T @ (np.exp(gam[-1] - gam)[:, None] * K)
    return out, S


def chunk_affine_map(k, v, g, beta):
    """(A, B) with S_out = S_in A + B for one chunk (used by the long-sequence path)."""
    n, dk = k.shape
    gam = np.cumsum(g)
    M = np.tril(np.exp(gam[:, None] - gam[None, :]))
    L = np.tril(beta[:, None] * M * (k @ k.T), -1)
    Tm = np.linalg.inv(np.eye(n) + L)
    W = Tm @ ((beta * np.exp(gam))[:, None] * k)
    Ut = Tm @ (beta[:, None] * v)
    D = np.exp(gam[-1] - gam)[:, None]
    return math.exp(gam[-1]) * np.eye(dk) - W.T @ (D * k), Ut.T @ (D * k)


def draw(seed, T, dk, dv, slow=False):
    r = np.random.default_rng(seed)
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    if slow:
        g = -r.uniform(1e-4, 2e-3, size=T)
    else:
        g = -math.exp(r.uniform(0, math.log(16))) * np.logaddexp(0, r.standard_normal(T) + 0.3)
    beta = 1 / (1 + np.exp(-r.standard_normal(T)))
    s0 = r.standard_normal((dv, dk)) * 0.1
    return q, k, v, g, beta, s0


@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 150])
@pytest.mark.parametrize("slow", [False, True])
def test_chunked_form_equals_recurrence(C, T, slow):
    q, k, v, g, beta, s0 = draw(T * 7 + C, T, 16, 12, slow)
    o_ref, s_ref, _ = oracle.forward(q[:, None], k[:, None], v[:, None], g[:, None],
                                     beta[:, None], s0[None, None], N=1)
    o, S = chunked(unit_rows(q), unit_rows(k), v, g, beta, s0, C)
    np.testing.assert_allclose(o, o_ref[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, s_ref[0, 0], rtol=0, atol=1e-12)


def test_affine_chunk_map_and_decay_bound():
    """S_out = S_in A + B holds exactly, and ||A||_2 <= exp(sum g) for 0 <= beta <= 1, |k| <= 1."""
    q, k, v, g, beta, s0 = draw(5, 64, 16, 12)
    kn = unit_rows(k)
    A, B = chunk_affine_map(kn, v, g, beta)
    _, s_ref, _ = oracle.forward(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                                 s0[None, None], N=1)
    np.testing.assert_allclose(s0 @ A + B, s_ref[0, 0], rtol=0, atol=1e-12)
    for slow in (False, True):
        q, k, v, g, beta, s0 = draw(6, 64, 16, 12, slow)
        A, _ = chunk_affine_map(unit_rows(k), v, g, beta)
        assert np.linalg.norm(A, 2) <= math.exp(g.sum()) * (1 + 1e-12)
