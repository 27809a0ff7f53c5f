"""Pins for the fp64 oracle: each test ties it to something other than itself.

Citations: the reading-notes page "PaTH Attention:通过累积 Householder 变换编码位置"
(cc.laoqi.cc), by section.

* brute-force d x d products of the definition            [s2.1]
* beta = 0 reduces to textbook causal softmax attention     [s2.1]
* beta = 0 with a forget gate reduces to the FoX bias form  [s2.5]
* empty path at i = j; position j's own transition excluded [s2.1]
* one transition changes only the w component, by 1 - beta  [s2.2]
* beta = 2 reflections preserve norms                       [s2.2]
* the printed swap / erase examples                         [s2.2]
* the printed permutation-score integers (55 vs <= 54)      [s2.4]
* the linear-RNN coefficients c_tj                          [s2.3]
* the cache rewrite identity (k_j^(t))^T q_t                [s2.8]

Every check here runs on the CPU.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(seed, S, L, d, dv=None, beta_mode="sigmoid"):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    q = rng.standard_normal((S, L, d))
    k = rng.standard_normal((S, L, d))
    v = rng.standard_normal((S, L, dv))
    w = rng.standard_normal((S, L, d))
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    if beta_mode == "sigmoid":
        beta = 2.0 / (1.0 + np.exp(-rng.standard_normal((S, L))))
    else:
        beta = np.full((S, L), float(beta_mode))
    logf = -np.log1p(np.exp(-(3.0 + rng.standard_normal((S, L)))))
    return q, k, v, w, beta, logf


def _transition(w, beta):
    d = w.shape[0]
    return np.eye(d) - beta * np.outer(w, w)


def _bruteforce_logits(q, k, w, beta, logf, scale):
    """Logits by explicit d x d products F_{j+1:i} = H_{j+1} ... H_i [s2.1]."""
    L, d = q.shape
    H = [_transition(w[t], beta[t]) for t in range(L)]
    A = np.full((L, L), -np.inf)
    for i in range(L):
        for j in range(i + 1):
            F = np.eye(d)
            for t in range(j + 1, i + 1):      # left-to-right: H_{j+1} ... H_i
                F = F @ H[t]
            A[i, j] = scale * (k[j] @ F @ q[i])
            if logf is not None:
                A[i, j] += logf[j + 1:i + 1].sum()   # sum_{s=j+1..i} log f_s [s2.5]
    return A


def _softmax_out(A, v):
    m = A.max(axis=1, keepdims=True)
    P = np.exp(A - m)
    l = P.sum(axis=1, keepdims=True)
    return (P / l) @ v, (m + np.log(l))[:, 0]


@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("shape", [(2, 9, 5), (1, 12, 3), (1, 1, 4)])
def test_walk_matches_bruteforce_products(fox, shape):
    S, L, d = shape
    q, k, v, w, beta, logf = _rand_inputs(11 + L + d, S, L, d)
    lf = logf if fox else None
    scale = 0.7
    o, lse = oracle.fwd_rows(q, k, v, w, beta, lf, scale)
    for s in range(S):
        A = _bruteforce_logits(q[s], k[s], w[s], beta[s], lf[s] if fox else None, scale)
        o_ref, lse_ref = _softmax_out(A, v[s])
        np.testing.assert_allclose(o[s], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[s], lse_ref, rtol=0, atol=1e-12)


def _raw_scores(q, k, w, beta, logf, scale):
    """Full logit matrix recovered from the oracle: one-hot values give A_ij."""
    S, L, _ = q.shape
    v = np.broadcast_to(np.eye(L), (S, L, L))
    P, lse = oracle.fwd_rows(q, k, v, w, beta, logf, scale)
    with np.errstate(divide="ignore"):
        return np.log(P) + lse[:, :, None]


def test_product_direction_matters():
    """Reversing the product order changes the logits: the pin above is sharp."""
    q, k, v, w, beta, _ = _rand_inputs(5, 1, 6, 4)
    A = _raw_scores(q, k, w, beta, None, 1.0)[0]
    H = [_transition(w[0, t], beta[0, t]) for t in range(6)]
    rev = k[0, 0] @ (H[5] @ H[4] @ H[3] @ H[2] @ H[1]) @ q[0, 5]
    fwd = k[0, 0] @ (H[1] @ H[2] @ H[3] @ H[4] @ H[5]) @ q[0, 5]
    assert abs(A[5, 0] - fwd) < 1e-12
    assert abs(rev - fwd) > 1e-3


def test_beta_zero_is_causal_softmax_attention():
    S, L, d = 3, 70, 16
    q, k, v, w, _, _ = _rand_inputs(3, S, L, d)
    beta = np.zeros((S, L))
    scale = d ** -0.5
    o, lse = oracle.fwd_rows(q, k, v, w, beta, None, scale)
    for s in range(S):
        A = scale * q[s] @ k[s].T
        A[np.triu_indices(L, 1)] = -np.inf
        o_ref, lse_ref = _softmax_out(A, v[s])
        np.testing.assert_allclose(o[s], o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[s], lse_ref, rtol=0, atol=1e-12)


def test_beta_zero_with_gate_is_forgetting_attention():
    S, L, d = 2, 40, 8
    q, k, v, w, _, logf = _rand_inputs(4, S, L, d)
    beta = np.zeros((S, L))
    o, lse = oracle.fwd_rows(q, k, v, w, beta, logf, 1.0)
    for s in range(S):
        c = np.cumsum(logf[s])                    # inclusive prefix C_i
        A = q[s] @ k[s].T + (c[:, None] - c[None, :])   # C_i - C_j = sum_{j<s<=i}
        A[np.triu_indices(L, 1)] = -np.inf
        o_ref, lse_ref = _softmax_out(A, v[s])
        np.testing.assert_allclose(o[s], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[s], lse_ref, rtol=0, atol=1e-12)


def test_zero_log_gate_equals_plain_path():
    q, k, v, w, beta, _ = _rand_inputs(6, 2, 30, 8)
    o1, l1 = oracle.fwd_rows(q, k, v, w, beta, None, 0.5)
    o2, l2 = oracle.fwd_rows(q, k, v, w, beta, np.zeros_like(beta), 0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_empty_path_on_the_diagonal_and_row_zero():
    """i = j: the path is empty, so the logit is scale * k_i . q_i [s2.1]."""
    S, L, d = 2, 25, 6
    q, k, v, w, beta, logf = _rand_inputs(7, S, L, d)
    scale = 0.3
    A = _raw_scores(q, k, w, beta, logf, scale)
    diag = scale * np.einsum("sld,sld->sl", q, k)
    np.testing.assert_allclose(np.diagonal(A, axis1=1, axis2=2), diag, atol=1e-12)
    o, lse = oracle.fwd_rows(q, k, v, w, beta, logf, scale, rows=[0])
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-15)
    np.testing.assert_allclose(lse[:, 0], diag[:, 0], atol=1e-15)


def test_first_transition_never_used_and_last_transition_used():
    """H_j is excluded from key j's path and H_i included [s2.1]."""
    q, k, v, w, beta, logf = _rand_inputs(8, 1, 20, 5)
    o1, l1 = oracle.fwd_rows(q, k, v, w, beta, logf, 1.0)
    w2, b2 = w.copy(), beta.copy()
    w2[:, 0] = np.eye(5)[1]
    b2[:, 0] = 1.7
    o2, l2 = oracle.fwd_rows(q, k, v, w2, b2, logf, 1.0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # changing the last position's transition does change the last row
    w3, b3 = w.copy(), beta.copy()
    b3[:, -1] = 0.0
    o3, _ = oracle.fwd_rows(q, k, v, w3, b3, logf, 1.0, rows=[19])
    assert np.abs(o3[:, 0] - o1[:, 19]).max() > 1e-6


def test_transition_changes_only_the_w_component():
    """H z = z_perp + (1 - beta) alpha w  [s2.2]; checked through the key walk."""
    rng = np.random.default_rng(9)
    d = 7
    for beta_val in [0.0, 0.3, 1.0, 1.5, 2.0]:
        k = rng.standard_normal((1, 2, d))
        w = rng.standard_normal((1, 2, d))
        w /= np.linalg.norm(w, axis=-1, keepdims=True)
        beta = np.full((1, 2), beta_val)
        out = oracle.transported_keys(k, w, beta, 1)[0, 0]   # H_1 k_0
        z, u = k[0, 0], w[0, 1]
        alpha = u @ z
        assert abs(u @ out - (1 - beta_val) * alpha) < 1e-14
        diff = out - z
        perp = diff - (diff @ u) * u
        assert np.abs(perp).max() < 1e-14


def test_reflections_preserve_norms():
    """beta = 2 makes every transition a reflection, so norms survive [s2.2]."""
    q, k, v, w, _, _ = _rand_inputs(10, 2, 200, 8)
    beta = np.full((2, 200), 2.0)
    out = oracle.transported_keys(k, w, beta, 199)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1),
                               np.linalg.norm(k, axis=-1), rtol=1e-12)
    # row scores equal k_j . (F q_i) with |F q_i| = |q_i|: bounded by Cauchy-Schwarz
    A = _raw_scores(q[:, :40], k[:, :40], w[:, :40], beta[:, :40], None, 1.0)
    bound = np.linalg.norm(q[:, :40], axis=-1)[:, :, None] * np.linalg.norm(k[:, :40], axis=-1)[:, None, :]
    low = np.tril(np.ones((40, 40), dtype=bool))
    assert np.all(np.abs(A[:, low]) <= bound[:, low] * (1 + 1e-12))


def test_printed_teaching_examples():
    g = json.load(open(os.path.join(GOLDEN, "householder_examples.json")))
    for case in g["cases"]:
        w = np.array(case["w"])
        M = np.array(case["matrix"])
        d = w.shape[0]
        # apply the single transition to each basis vector via the cache walk
        for e in range(d):
            k = np.zeros((1, 2, d))
            k[0, 0] = np.eye(d)[e]
            W = np.zeros((1, 2, d))
            W[0, 1] = w
            beta = np.array([[0.0, case["beta"]]])
            col = oracle.transported_keys(k, W, beta, 1)[0, 0]
            np.testing.assert_allclose(col, M[:, e], atol=1e-15)


def _compose(n_elem, swaps):
    """Track the permutation combinatorially (no linear algebra)."""
    pos = list(range(1, n_elem + 1))
    for a, b in swaps:
        pos[a], pos[b] = pos[b], pos[a]
    return pos


def test_printed_permutation_scores():
    g = json.load(open(os.path.join(GOLDEN, "permutation_score.json")))["facts"]
    n = g["elements"]
    rng = np.random.default_rng(12)
    seen_identity = seen_other = 0
    for trial in range(60):
        m = int(rng.integers(1, 9))
        if trial % 3 == 0:      # force identities: a sequence followed by its reverse
            half = [tuple(rng.choice(n, 2, replace=False)) for _ in range(m)]
            swaps = half + half[::-1]
        else:
            swaps = [tuple(rng.choice(n, 2, replace=False)) for _ in range(m)]
        L = len(swaps) + 1
        q = np.zeros((1, L, n))
        k = np.zeros((1, L, n))
        w = np.zeros((1, L, n))
        beta = np.zeros((1, L))
        k[0, 0] = np.arange(1, n + 1)
        q[0, L - 1] = np.arange(1, n + 1)
        for t, (a, b) in enumerate(swaps, start=1):
            w[0, t, a], w[0, t, b] = 2 ** -0.5, -(2 ** -0.5)
            beta[0, t] = 2.0
        v = np.zeros((1, L, 1))
        _, lse = oracle.fwd_rows(q, k, v, w, beta, None, 1.0, rows=[L - 1])
        # key 0 carries s0; the L-1 other keys score exactly 0
        s0 = lse[0, 0] + np.log1p(-(L - 1) * np.exp(-lse[0, 0]))
        perm = _compose(n, swaps)
        total = sum(r * p for r, p in zip(range(1, n + 1), perm))
        assert abs(s0 - total) < 1e-9
        if perm == list(range(1, n + 1)):
            assert round(s0) == g["identity_sum"]
            seen_identity += 1
        else:
            assert s0 <= g["non_identity_max_sum"] + 1e-9
            assert s0 < g["threshold"]
            seen_other += 1
    assert seen_identity > 5 and seen_other > 5


def test_linear_rnn_coefficients():
    """S_t = S_{t-1} H_t + v_t k_t^T with one-hot v_t gives c_tj [s2.3]."""
    S_, L, d = 1, 14, 5
    q, k, _, w, beta, _ = _rand_inputs(13, S_, L, d)
    A = _raw_scores(q, k, w, beta, None, 1.0)[0]
    state = np.zeros((L, d))
    for t in range(L):
        H = np.eye(d) - beta[0, t] * np.outer(w[0, t], w[0, t])
        state = state @ H
        state[t] += k[0, t]                       # v_t = e_t
        c = state @ q[0, t]                       # o_t = S_t q_t
        np.testing.assert_allclose(A[t, :t + 1], c[:t + 1], atol=1e-12)


def test_cache_rewrite_identity():
    """(k_j^(t))^T q_t = k_j^T H_{j+1}...H_t q_t: rewritten keys give row t [s2.8]."""
    q, k, _, w, beta, logf = _rand_inputs(14, 2, 30, 6)
    A = _raw_scores(q, k, w, beta, None, 1.0)
    for t in [0, 1, 17, 29]:
        kt = oracle.transported_keys(k, w, beta, t)
        scores = np.einsum("sjd,sd->sj", kt, q[:, t])
        np.testing.assert_allclose(scores, A[:, t, :t + 1], atol=1e-12)
    # and against explicit products
    kt = oracle.transported_keys(k, w, beta, 29)
    for j in [0, 5, 28, 29]:
        z = k[0, j].copy()
        M = np.eye(6)
        for s in range(j + 1, 30):
            M = _transition(w[0, s], beta[0, s]) @ M     # H_t ... H_{j+1}
        np.testing.assert_allclose(kt[0, j], M @ z, atol=1e-12)


def test_softmax_invariants():
    q, k, v, w, beta, logf = _rand_inputs(15, 2, 50, 8)
    L = 50
    P, lse = oracle.fwd_rows(q, k, np.broadcast_to(np.eye(L), (2, L, L)), w, beta, logf, 1.0)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-13)
    assert np.all(np.triu(P[0], 1) == 0)
    A = _raw_scores(q, k, w, beta, logf, 1.0)
    assert np.all(lse >= np.nanmax(np.where(np.isfinite(A), A, -np.inf), axis=-1) - 1e-12)


def test_rows_out_of_range_rejected():
    q, k, v, w, beta, _ = _rand_inputs(1, 1, 4, 2)
    with pytest.raises(ValueError):
        oracle.fwd_rows(q, k, v, w, beta, None, 1.0, rows=[4])
