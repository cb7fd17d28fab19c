"""Pins of the fp64 oracle against facts the pages and the mathematics fix (CPU only).

Each test is chosen so that a plausible mistake in the oracle (a dropped term, a wrong sign,
a transposed operand, a decay applied to the write, a conv tap reversed, a leak across
sequences) fails at least one of them.  None of these re-types the oracle's loop: expected
values come from a hand-worked example, closed forms, explicit matrix products of the printed
rule, special cases and numpy library routines.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed):
    return np.random.default_rng(seed)


def unit_rows(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


def gates(r, T, H, slow=False):
    if slow:
        g = -r.uniform(1e-4, 2e-3, size=(T, H))
    else:
        g = -np.exp(r.uniform(0, math.log(16), size=H))[None] * np.logaddexp(
            0, r.standard_normal((T, H)) + r.normal(0, 0.5, size=H)[None])
    beta = 1 / (1 + np.exp(-r.standard_normal((T, H))))
    return g, beta


def transition_products(q, k, v, g, beta, s0, scale=1.0):
    """States and outputs from the rule as printed: explicit dk x dk transition matrices
    A_t = alpha_t (I - beta_t k_t k_t^T) and S_t = S_{t-1} A_t + beta_t v_t k_t^T."""
    T, dk = k.shape
    S = s0.copy()
    outs = []
    for t in range(T):
        A = math.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t]))
        S = S @ A + beta[t] * np.outer(v[t], k[t])
        outs.append(scale * S @ q[t])
    return np.array(outs), S


def unrolled_sum(k, v, g, beta, s0):
    """Final state by the unrolled sum S_T = S0 prod_t A_t + sum_t beta_t v_t k_t^T prod_{s>t} A_s."""
    T, dk = k.shape
    A = [math.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    P = np.eye(dk)
    for t in range(T):
        P = P @ A[t]
    S = s0 @ P
    for t in range(T):
        P = np.eye(dk)
        for s in range(t + 1, T):
            P = P @ A[s]
        S = S + beta[t] * np.outer(v[t], k[t]) @ P
    return S


def one_head(q, k, v, g, beta, s0=None, **kw):
    """Run the oracle on a single (sequence, head) given [T, d] arrays."""
    T, dk = q.shape
    dv = v.shape[1]
    s0a = None if s0 is None else s0[None, None]
    o, sf, _ = oracle.forward(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                              s0a, None, None, N=1, **kw)
    return o[:, 0], sf[0, 0]


# --------------------------------------------------------------------------------------------

def test_hand_worked_example():
    """Pencil-and-paper values (tests/golden/hand_worked_dk2.txt), exact in fp64."""
    d = {}
    for line in open(os.path.join(GOLDEN, "hand_worked_dk2.txt")):
        if line.startswith("#") or ":" not in line:
            continue
        key, vals = line.split(":", 1)
        d[key.strip()] = np.array([float(x) for x in vals.split()])
    o, sf = one_head(d["q"].reshape(3, 2), d["k"].reshape(3, 2), d["v"].reshape(3, 2), d["g"],
                     d["beta"], d["S0"].reshape(2, 2), l2norm=False)
    np.testing.assert_array_equal(o.reshape(-1), d["o"])
    np.testing.assert_array_equal(sf.reshape(-1), d["S_final"])


@pytest.mark.parametrize("l2norm", [False, True])
def test_matches_explicit_transition_products(l2norm):
    """The oracle equals the printed rule evaluated with explicit matrices (tiny sizes)."""
    r = rnd(1)
    T, dk, dv = 9, 5, 3
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    g, beta = gates(r, T, 1)
    g, beta = g[:, 0] * 0.1, beta[:, 0]
    s0 = r.standard_normal((dv, dk))
    o, sf = one_head(q, k, v, g, beta, s0, l2norm=l2norm, scale=0.7)
    qn, kn = (unit_rows(q), unit_rows(k)) if l2norm else (q, k)
    o_ref, s_ref = transition_products(qn, kn, v, g, beta, s0, scale=0.7)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, s_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, unrolled_sum(kn, v, g, beta, s0), rtol=0, atol=1e-13)


def test_beta_zero_is_pure_decay():
    """beta = 0: S_t = exp(sum g) S_0 and o_t = exp(gamma_t) S_0 q_t (decay only)."""
    r = rnd(2)
    T, dk, dv = 40, 8, 6
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    g = -r.uniform(0, 0.3, size=T)
    s0 = r.standard_normal((dv, dk))
    o, sf = one_head(q, k, v, g, np.zeros(T), s0)
    gam = np.cumsum(g)
    np.testing.assert_allclose(sf, math.exp(gam[-1]) * s0, rtol=1e-12)
    np.testing.assert_allclose(o, np.exp(gam)[:, None] * (unit_rows(q) @ s0.T), rtol=1e-11,
                               atol=1e-14)


def test_alpha_one_beta_zero_keeps_state_bitwise():
    r = rnd(3)
    T, dk, dv = 17, 8, 8
    s0 = r.standard_normal((dv, dk))
    q = r.standard_normal((T, dk))
    o, sf = one_head(q, r.standard_normal((T, dk)), r.standard_normal((T, dv)), np.zeros(T),
                     np.zeros(T), s0)
    np.testing.assert_array_equal(sf, s0)
    np.testing.assert_allclose(o, unit_rows(q) @ s0.T, rtol=1e-14, atol=1e-15)


def test_beta_one_retrieves_the_written_value():
    """beta = 1 with unit keys overwrites the slot: S_t k_t = v_t.  With q = k the read-out is
    o_t = S_t k_t, so o must equal v (up to the eps of the L2 norm, taken off here)."""
    r = rnd(4)
    T, dk, dv = 30, 16, 8
    k = unit_rows(r.standard_normal((T, dk)))
    k = k / np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    g, _ = gates(r, T, 1)
    o, _ = one_head(k, k, v, g[:, 0], np.ones(T), r.standard_normal((dv, dk)), l2norm=False)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_single_step_is_sgd_with_weight_decay():
    """Page 发现一, online-learning view: S_t = S' - beta grad_S 1/2 ||S k - v||^2 at S' = alpha
    S_{t-1}, grad = (S' k - v) k^T.  Non-symmetric S catches a transposed product."""
    r = rnd(5)
    dk, dv = 7, 5
    s0 = r.standard_normal((dv, dk))
    q, k, v = r.standard_normal((1, dk)), r.standard_normal((1, dk)), r.standard_normal((1, dv))
    g, b = np.array([-0.37]), np.array([0.61])
    _, sf = one_head(q, k, v, g, b, s0, l2norm=False)
    sp = math.exp(g[0]) * s0
    grad = np.outer(sp @ k[0] - v[0], k[0])
    np.testing.assert_allclose(sf, sp - b[0] * grad, rtol=0, atol=1e-14)


def test_g_zero_is_deltanet():
    """g = 0 reduces to the DeltaNet rule S_t = S_{t-1}(I - beta k k^T) + beta v k^T (page
    发现一, second bullet), evaluated here with explicit matrices."""
    r = rnd(6)
    T, dk, dv = 12, 6, 4
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    beta = r.uniform(0, 1, size=T)
    s0 = r.standard_normal((dv, dk))
    _, sf = one_head(q, k, v, np.zeros(T), beta, s0)
    kn = unit_rows(k)
    S = s0.copy()
    for t in range(T):
        S = S @ (np.eye(dk) - beta[t] * np.outer(kn[t], kn[t])) + beta[t] * np.outer(v[t], kn[t])
    np.testing.assert_allclose(sf, S, rtol=0, atol=1e-13)


def test_alpha_to_zero_empties_the_state():
    """alpha -> 0 (g = -1000, exp underflows to exactly 0): the old state is wiped and
    S_t = beta_t v_t k_t^T (page "Gated DeltaNet 架构详解...", section 6)."""
    r = rnd(7)
    T, dk, dv = 5, 4, 3
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    beta = r.uniform(0.1, 1, size=T)
    o, sf = one_head(q, k, v, np.full(T, -1000.0), beta, r.standard_normal((dv, dk)))
    qn, kn = unit_rows(q), unit_rows(k)
    np.testing.assert_allclose(sf, beta[-1] * np.outer(v[-1], kn[-1]), rtol=1e-14)
    np.testing.assert_allclose(o, beta[:, None] * v * (qn * kn).sum(1)[:, None], rtol=1e-13)


def test_one_hot_keys_closed_form():
    """One-hot keys decouple the key slots: slot j of S follows the scalar EMA
    s <- alpha s off-slot and s <- alpha (1 - beta) s + beta v on-slot.  Dyadic gates keep
    every operation exact, so equality is bitwise."""
    r = rnd(8)
    T, dk, dv = 24, 8, 4  # short enough that every mantissa stays within 53 bits
    slots = r.integers(0, dk, size=T)
    reads = r.integers(0, dk, size=T)
    k = np.eye(dk)[slots]
    q = np.eye(dk)[reads]
    v = r.integers(-8, 9, size=(T, dv)).astype(float)
    alpha = r.choice([1.0, 0.5, 0.25], size=T)
    beta = r.choice([0.0, 0.25, 0.5, 1.0], size=T)
    s0 = r.integers(-4, 5, size=(dv, dk)).astype(float)
    o, sf = one_head(q, k, v, np.log(alpha), beta, s0, l2norm=False)
    S = s0.copy()
    exp_o = []
    for t in range(T):
        for j in range(dk):
            if j == slots[t]:
                S[:, j] = alpha[t] * (1 - beta[t]) * S[:, j] + beta[t] * v[t]
            else:
                S[:, j] = alpha[t] * S[:, j]
        exp_o.append(S[:, reads[t]].copy())
    np.testing.assert_array_equal(sf, S)
    np.testing.assert_array_equal(o, np.array(exp_o))


def test_l2norm_definition():
    """The in-oracle L2 norm is x / sqrt(sum x^2 + 1e-6): running on raw inputs with the flag
    equals running on numpy-normalised inputs without it."""
    r = rnd(9)
    T, dk, dv = 20, 16, 8
    q, k, v = r.standard_normal((T, dk)) * 3, r.standard_normal((T, dk)) * 0.01, r.standard_normal((T, dv))
    g, beta = gates(r, T, 1)
    s0 = r.standard_normal((dv, dk))
    o1, s1 = one_head(q, k, v, g[:, 0], beta[:, 0], s0, l2norm=True)
    o2, s2 = one_head(unit_rows(q), unit_rows(k), v, g[:, 0], beta[:, 0], s0, l2norm=False)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-15)


def test_linear_in_values_and_initial_state():
    """For fixed q, k, g, beta the map (V, S_0) -> (O, S_T) is linear."""
    r = rnd(10)
    T, dk, dv = 33, 8, 8
    q, k = r.standard_normal((T, dk)), r.standard_normal((T, dk))
    v1, v2 = r.standard_normal((T, dv)), r.standard_normal((T, dv))
    s1, s2 = r.standard_normal((dv, dk)), r.standard_normal((dv, dk))
    g, beta = gates(r, T, 1, slow=True)
    o1, f1 = one_head(q, k, v1, g[:, 0], beta[:, 0], s1)
    o2, f2 = one_head(q, k, v2, g[:, 0], beta[:, 0], s2)
    o3, f3 = one_head(q, k, 2 * v1 - 3 * v2, g[:, 0], beta[:, 0], 2 * s1 - 3 * s2)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f3, 2 * f1 - 3 * f2, rtol=0, atol=1e-12)


def test_causal():
    """Changing tokens after t leaves o_<=t bitwise unchanged."""
    r = rnd(11)
    T, dk, dv = 20, 8, 8
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    g, beta = gates(r, T, 1)
    o1, _ = one_head(q, k, v, g[:, 0], beta[:, 0])
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[12:] += 1
    k2[12:] -= 1
    v2[12:] *= 3
    o2, _ = one_head(q2, k2, v2, g[:, 0], beta[:, 0])
    np.testing.assert_array_equal(o1[:12], o2[:12])
    assert not np.allclose(o1[12:], o2[12:])


def _pack(r, lengths, H, dk, dv):
    T = int(sum(lengths))
    q, k, v = r.standard_normal((T, H, dk)), r.standard_normal((T, H, dk)), r.standard_normal((T, H, dv))
    g, beta = gates(r, T, H)
    s0 = r.standard_normal((len(lengths), H, dv, dk)) * 0.1
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return q, k, v, g, beta, s0, cu


def test_varlen_packing_equals_separate_calls():
    r = rnd(12)
    lengths = [5, 0, 17, 1, 9]
    H, dk, dv = 3, 8, 4
    q, k, v, g, beta, s0, cu = _pack(r, lengths, H, dk, dv)
    o, sf, _ = oracle.forward(q, k, v, g, beta, s0, cu)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        on, sn, _ = oracle.forward(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0[n:n + 1], N=1)
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(sf[n], sn[0])
    # zero-length sequence: final state = initial state
    np.testing.assert_array_equal(sf[1], s0[1])


def test_split_and_resume():
    r = rnd(13)
    H, dk, dv = 2, 8, 8
    q, k, v, g, beta, s0, _ = _pack(r, [50], H, dk, dv)
    o, sf, _ = oracle.forward(q, k, v, g, beta, s0, N=1)
    _, s_mid, _ = oracle.forward(q[:23], k[:23], v[:23], g[:23], beta[:23], s0, N=1)
    o2, sf2, _ = oracle.forward(q[23:], k[23:], v[23:], g[23:], beta[23:], s_mid, N=1)
    np.testing.assert_array_equal(o[23:], o2)
    np.testing.assert_array_equal(sf, sf2)


def test_step_is_forward_with_one_token():
    r = rnd(14)
    N, H, dk, dv = 6, 3, 8, 4
    q, k, v = r.standard_normal((N, H, dk)), r.standard_normal((N, H, dk)), r.standard_normal((N, H, dv))
    g, beta = gates(r, N, H)
    st = r.standard_normal((N, H, dv, dk))
    o, st2 = oracle.step(q, k, v, g, beta, st, scale=0.5)
    o_ref, s_ref, _ = oracle.forward(q, k, v, g, beta, st, N=N, scale=0.5)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(st2, s_ref)


def test_subset_of_pairs_matches_full_run():
    r = rnd(15)
    H, dk, dv = 4, 8, 8
    q, k, v, g, beta, s0, cu = _pack(r, [7, 11], H, dk, dv)
    o, sf, _ = oracle.forward(q, k, v, g, beta, s0, cu)
    o2, sf2, _ = oracle.forward(q, k, v, g, beta, s0, cu, pairs=[(1, 2), (0, 3)])
    np.testing.assert_array_equal(o2[7:, 2], o[7:, 2])
    np.testing.assert_array_equal(o2[:7, 3], o[:7, 3])
    np.testing.assert_array_equal(sf2[1, 2], sf[1, 2])
    assert np.isnan(sf2[0, 0]).all()


def _conv_ref(x, w):
    """Causal 4-tap conv by numpy.convolve (tap 3 = current token), then SiLU."""
    y = np.convolve(x, w[::-1])[: len(x)]
    return y / (1 + np.exp(-y))


def test_conv_prologue_matches_numpy_convolve():
    """With alpha = 0 (g = -1000) and beta = 1, S_t = v'_t k'_t^T, so with identical q and k
    channels o_t = v'_t * |k'_t|^2 / (|k'_t|^2 + eps): the conv+SiLU output of v is read back
    directly.  Two packed sequences check zero history at each sequence start."""
    r = rnd(16)
    lengths = [6, 9]
    H, dk, dv = 2, 4, 3
    T = sum(lengths)
    x = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    wq = r.normal(0, 0.5, size=(H * dk, 4))
    wv = r.normal(0, 0.5, size=(H * dv, 4))
    conv_w = np.concatenate([wq, wq, wv])
    cu = np.array([0, 6, 15])
    o, sf, _ = oracle.forward(x, x, v, np.full((T, H), -1000.0), np.ones((T, H)), None, cu, conv_w)
    for n in range(2):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            kp = np.stack([_conv_ref(x[a:b, h, i], wq[h * dk + i]) for i in range(dk)], 1)
            vp = np.stack([_conv_ref(v[a:b, h, i], wv[h * dv + i]) for i in range(dv)], 1)
            n2 = (kp * kp).sum(1)
            np.testing.assert_allclose(o[a:b, h], vp * (n2 / (n2 + 1e-6))[:, None], rtol=1e-12,
                                       atol=1e-15)
            kn = kp[-1] / math.sqrt(n2[-1] + 1e-6)
            np.testing.assert_allclose(sf[n, h], np.outer(vp[-1], kn), rtol=1e-12, atol=1e-15)


def test_conv_single_tap_shifts():
    """Tap j alone delays the channel by 3 - j tokens (zeros before the sequence start)."""
    T, H, dk, dv = 8, 1, 2, 2
    r = rnd(17)
    x = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    for j in range(4):
        w = np.zeros((H * (2 * dk + dv), 4))
        w[:, j] = 1.0
        o, _, _ = oracle.forward(x, x, v, np.full((T, H), -1000.0), np.ones((T, H)), None,
                                 np.array([0, T]), w, l2norm=False)
        lag = 3 - j
        vs = np.zeros_like(v[:, 0])
        vs[lag:] = v[: T - lag, 0]
        xs = np.zeros_like(x[:, 0])
        xs[lag:] = x[: T - lag, 0]
        silu = lambda z: z / (1 + np.exp(-z))
        exp_o = silu(vs) * (silu(xs) ** 2).sum(1, keepdims=True)
        np.testing.assert_allclose(o[:, 0], exp_o, rtol=1e-13, atol=1e-300)


def test_gates_formula():
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b) (page maplevalley.com.cn,
    section 2.1), against closed-form points and numpy's logaddexp."""
    a = np.array([[0.0, 50.0, -50.0, 1.3]])
    b = np.array([[0.0, 3.0, -3.0, 0.7]])
    A_log = np.array([0.0, math.log(2), math.log(16), 0.3])
    dt = np.array([0.0, 0.0, 0.0, -0.2])
    g, beta = oracle.gates(a, b, A_log, dt)
    assert g[0, 0] == -math.log(2)
    assert beta[0, 0] == 0.5
    np.testing.assert_allclose(g[0], -np.exp(A_log) * np.logaddexp(0, a[0] + dt), rtol=1e-15)
    np.testing.assert_allclose(g[0, 2], -16 * math.exp(-50), rtol=1e-14)
    np.testing.assert_allclose(beta[0], 1 / (1 + np.exp(-b[0])), rtol=1e-15)


def _raw_rows(q, k, v):
    """Token rows of the conv channels in the order [q heads, k heads, v heads]."""
    T = q.shape[0]
    return np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], 1)


def test_conv_history_matches_numpy_convolve():
    """A given conv history acts as the three raw tokens before the sequence: the read-back of
    the conv+SiLU output of v (alpha = 0, beta = 1, q = k) equals numpy.convolve over the
    history followed by the sequence, with the history positions dropped."""
    r = rnd(18)
    lengths = [5, 2, 7]
    H, dk, dv = 2, 4, 3
    T = sum(lengths)
    C = H * (2 * dk + dv)
    x = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    wq = r.normal(0, 0.5, size=(H * dk, 4))
    wv = r.normal(0, 0.5, size=(H * dv, 4))
    conv_w = np.concatenate([wq, wq, wv])
    hist = r.standard_normal((3, 3, C))
    hist[:, :, H * dk:2 * H * dk] = hist[:, :, :H * dk]   # k history = q history (q = k)
    cu = np.array([0, 5, 7, 14])
    o, sf, _ = oracle.forward(x, x, v, np.full((T, H), -1000.0), np.ones((T, H)), None, cu, conv_w,
                              conv_hist=hist)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            kcols = [np.concatenate([hist[n, :, h * dk + i], x[a:b, h, i]]) for i in range(dk)]
            vcols = [np.concatenate([hist[n, :, 2 * H * dk + h * dv + i], v[a:b, h, i]]) for i in range(dv)]
            kp = np.stack([_conv_ref(c, wq[h * dk + i])[3:] for i, c in enumerate(kcols)], 1)
            vp = np.stack([_conv_ref(c, wv[h * dv + i])[3:] for i, c in enumerate(vcols)], 1)
            n2 = (kp * kp).sum(1)
            np.testing.assert_allclose(o[a:b, h], vp * (n2 / (n2 + 1e-6))[:, None], rtol=1e-12,
                                       atol=1e-15)


def test_conv_history_out_is_last_three_raw_tokens():
    """The history after a sequence is, by definition, its last three raw inputs, continued from
    the history before it when the sequence is shorter than three (zero length keeps it)."""
    r = rnd(19)
    lengths = [0, 1, 2, 3, 6]
    H, dk, dv = 2, 4, 2
    q, k, v, g, beta, s0, cu = _pack(r, lengths, H, dk, dv)
    C = H * (2 * dk + dv)
    conv_w = r.normal(0, 0.5, size=(C, 4))
    hist = r.standard_normal((len(lengths), 3, C))
    _, _, _, hout = oracle.forward(q, k, v, g, beta, s0, cu, conv_w, conv_hist=hist,
                                   want_conv_hist=True)
    raw = _raw_rows(q, k, v)
    for n in range(len(lengths)):
        seq = np.concatenate([hist[n], raw[cu[n]:cu[n + 1]]])
        np.testing.assert_array_equal(hout[n], seq[-3:])
    # without a history the rows before the sequence are zeros
    _, _, _, hz = oracle.forward(q, k, v, g, beta, s0, cu, conv_w, want_conv_hist=True)
    np.testing.assert_array_equal(hz[1], np.concatenate([np.zeros((2, C)), raw[0:1]]))


def test_conv_split_and_resume():
    """One sequence run whole equals its first part followed by the rest, the second part given
    the state and the conv history the first one left (split points inside the conv window)."""
    r = rnd(20)
    H, dk, dv = 2, 8, 4
    q, k, v, g, beta, s0, _ = _pack(r, [40], H, dk, dv)
    conv_w = r.normal(0, 0.5, size=(H * (2 * dk + dv), 4))
    o, sf, _, hf = oracle.forward(q, k, v, g, beta, s0, None, conv_w, N=1, want_conv_hist=True)
    for cut in (1, 2, 17):
        o1, s1, _, h1 = oracle.forward(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], s0, None,
                                       conv_w, N=1, want_conv_hist=True)
        o2, s2, _, h2 = oracle.forward(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], s1, None,
                                       conv_w, N=1, conv_hist=h1, want_conv_hist=True)
        np.testing.assert_array_equal(o[:cut], o1)
        np.testing.assert_array_equal(o[cut:], o2)
        np.testing.assert_array_equal(sf, s2)
        np.testing.assert_array_equal(hf, h2)


def test_step_with_conv_is_forward_last_token():
    """A decode step with conv, given the state and history after T - 1 tokens, reproduces the
    last token of the whole-sequence forward pass, and its history equals the forward pass's."""
    r = rnd(21)
    lengths = [9, 4, 12]
    H, dk, dv = 2, 8, 4
    q, k, v, g, beta, s0, cu = _pack(r, lengths, H, dk, dv)
    C = H * (2 * dk + dv)
    conv_w = r.normal(0, 0.5, size=(C, 4))
    hist = r.standard_normal((3, 3, C))
    o, sf, _, hf = oracle.forward(q, k, v, g, beta, s0, cu, conv_w, conv_hist=hist,
                                  want_conv_hist=True)
    last = cu[1:] - 1
    keep = np.ones(cu[-1], bool)
    keep[last] = False
    cu_head = cu - np.arange(len(cu))
    _, s_h, _, h_h = oracle.forward(q[keep], k[keep], v[keep], g[keep], beta[keep], s0, cu_head,
                                    conv_w, conv_hist=hist, want_conv_hist=True)
    o_s, s_s, h_s = oracle.step(q[last], k[last], v[last], g[last], beta[last], s_h,
                                conv_w=conv_w, conv_hist=h_h)
    np.testing.assert_array_equal(o_s, o[last])
    np.testing.assert_array_equal(s_s, sf)
    np.testing.assert_array_equal(h_s, hf)


def _expand_heads(x, r):
    """[T, Hk, d] -> [T, Hk * r, d], each query/key head repeated for its r value heads."""
    return np.repeat(x, r, axis=1)


def _expand_conv_rows(w, Hk, r, dk, H, dv):
    """Conv channels (rows of a [C, ...] array) of the grouped layout 2*Hk*dk + H*dv mapped to the
    layout with one query/key head per value head (2*H*dk + H*dv)."""
    q = w[:Hk * dk].reshape(Hk, dk, *w.shape[1:])
    k = w[Hk * dk:2 * Hk * dk].reshape(Hk, dk, *w.shape[1:])
    v = w[2 * Hk * dk:]
    return np.concatenate([np.repeat(q, r, 0).reshape(H * dk, *w.shape[1:]),
                           np.repeat(k, r, 0).reshape(H * dk, *w.shape[1:]), v])


@pytest.mark.parametrize("Hk,H", [(1, 3), (2, 4), (3, 3)])
def test_grouped_heads_equal_repeated_heads(Hk, H):
    """Value heads sharing a query/key head: the result equals the one-to-one layout with every
    query/key head (and its conv weights and history) repeated for the value heads that use it.
    Bitwise, with the conv prologue, a history in and out, and a decode step."""
    r = rnd(22 + Hk + H)
    rep = H // Hk
    lengths = [9, 0, 2, 14]
    dk, dv = 4, 3
    T = sum(lengths)
    q, k = r.standard_normal((T, Hk, dk)), r.standard_normal((T, Hk, dk))
    v = r.standard_normal((T, H, dv))
    g, beta = gates(r, T, H)
    s0 = r.standard_normal((len(lengths), H, dv, dk)) * 0.1
    cu = np.concatenate([[0], np.cumsum(lengths)])
    C = 2 * Hk * dk + H * dv
    conv_w = r.normal(0, 0.5, size=(C, 4))
    hist = r.standard_normal((len(lengths), 3, C))
    o, sf, _, hf = oracle.forward(q, k, v, g, beta, s0, cu, conv_w, conv_hist=hist, want_conv_hist=True)
    ew = _expand_conv_rows(conv_w, Hk, rep, dk, H, dv)
    eh = np.ascontiguousarray(np.stack([_expand_conv_rows(hist[n].T, Hk, rep, dk, H, dv).T
                                        for n in range(len(lengths))]))
    o2, sf2, _, hf2 = oracle.forward(_expand_heads(q, rep), _expand_heads(k, rep), v, g, beta, s0, cu, ew,
                                     conv_hist=eh, want_conv_hist=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(sf, sf2)
    for n in range(len(lengths)):
        np.testing.assert_array_equal(_expand_conv_rows(hf[n].T, Hk, rep, dk, H, dv).T, hf2[n])
    # decode step
    N = 5
    qd, kd = r.standard_normal((N, Hk, dk)), r.standard_normal((N, Hk, dk))
    vd = r.standard_normal((N, H, dv))
    gd, bd = gates(r, N, H)
    st = r.standard_normal((N, H, dv, dk))
    hd = r.standard_normal((N, 3, C))
    od, std, hdo = oracle.step(qd, kd, vd, gd, bd, st, conv_w=conv_w, conv_hist=hd)
    ehd = np.ascontiguousarray(np.stack([_expand_conv_rows(hd[n].T, Hk, rep, dk, H, dv).T for n in range(N)]))
    od2, std2, hdo2 = oracle.step(_expand_heads(qd, rep), _expand_heads(kd, rep), vd, gd, bd, st, conv_w=ew,
                                  conv_hist=ehd)
    np.testing.assert_array_equal(od, od2)
    np.testing.assert_array_equal(std, std2)
    for n in range(N):
        np.testing.assert_array_equal(_expand_conv_rows(hdo[n].T, Hk, rep, dk, H, dv).T, hdo2[n])


# -------------------------------------------------------------------------- output epilogue

def test_gated_norm_hand_worked():
    """o = (3, 4): mean square 12.5; w = (0, 1) gives scales (1, 2); z = 0 gives sigmoid 1/2."""
    out = oracle.gated_norm(np.array([[3.0, 4.0]]), np.zeros((1, 2)), np.array([0.0, 1.0]), 0.0)
    np.testing.assert_allclose(out[0], [3 / (2 * math.sqrt(12.5)), 4 / math.sqrt(12.5)], rtol=1e-15)


def test_gated_norm_properties():
    r = rnd(23)
    o = r.standard_normal((7, 3, 16))
    z = r.standard_normal(o.shape)
    w = r.normal(0, 0.3, size=16)
    # an open gate (sigmoid(40) = 1 in fp64) and w = 0: unit root mean square per row (eps = 0)
    out = oracle.gated_norm(o, np.full(o.shape, 40.0), np.zeros(16), 0.0)
    np.testing.assert_allclose(np.sqrt((out ** 2).mean(-1)), 1.0, rtol=1e-14)
    # z = 0 halves the open-gate output exactly
    half = oracle.gated_norm(o, np.zeros(o.shape), w, 1e-3)
    full = oracle.gated_norm(o, np.full(o.shape, 40.0), w, 1e-3)
    np.testing.assert_array_equal(half * 2, full)
    # invariant under a positive rescaling of o when eps = 0
    np.testing.assert_allclose(oracle.gated_norm(5.5 * o, z, w, 0.0), oracle.gated_norm(o, z, w, 0.0), rtol=1e-13)
    # w = -1 closes every channel
    assert not oracle.gated_norm(o, z, -np.ones(16), 1e-3).any()
    # eps enters as mean(o^2) + eps: a row of zeros except o0 = 1, dv = 16, eps = 1/16 -> o0 / sqrt(1/8)
    e = np.zeros((1, 16))
    e[0, 0] = 1.0
    out = oracle.gated_norm(e, np.full(e.shape, 40.0), np.zeros(16), 1.0 / 16)
    assert out[0, 0] == pytest.approx(math.sqrt(8.0), rel=1e-15)
