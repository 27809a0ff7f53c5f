"""Pins of the backward oracle (oracle.bwd): gradients of sum(do * o).

The pages give no backward formulas, so the oracle's gradients are the
reverse-mode derivative of its forward walk.  They are pinned here by
quantities that do not go through that derivation:
  * central finite differences of the forward oracle (fwd_rows), for every
    input, with and without the forget gate;
  * beta = 0 without a gate: the textbook softmax-attention gradients for q,
    k and v, zero for w, and a closed form for beta (all transitions are the
    identity there, so the walk's vectors are the raw queries and keys);
  * the first position's w, beta and log f never reach an output (the path
    of a pair j <= i holds H_{j+1} .. H_i, the bias log f_{j+1} .. log f_i),
    so their gradients are exactly zero;
  * each of several planted mistakes in a copy of the oracle makes the
    finite-difference pin fail.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _rand_inputs

SCALE = 0.7


def _loss(orc, q, k, v, w, beta, logf, do):
    o, _ = orc.fwd_rows(q, k, v, w, beta, logf, SCALE)
    return float(np.sum(o * do))


def _fd_grads(orc, args, names, h=1e-5):
    """Central differences of sum(do * o) for each named input array."""
    out = {}
    for name in names:
        x = args[name]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(orc, **args)
            x[idx] = keep - h
            lm = _loss(orc, **args)
            x[idx] = keep
            g[idx] = (lp - lm) / (2 * h)
        out[name] = g
    return out


def _case(seed, gate, S=2, L=6, d=3, dv=2):
    q, k, v, w, beta, logf = _rand_inputs(seed, S, L, d, dv)
    rng = np.random.default_rng(seed + 100)
    do = rng.standard_normal((S, L, dv))
    return dict(q=q, k=k, v=v, w=w, beta=beta, logf=logf if gate else None, do=do)


def _fd_matches(orc, args):
    g = orc.bwd(args["q"], args["k"], args["v"], args["w"], args["beta"], args["logf"],
                SCALE, args["do"])
    names = ["q", "k", "v", "w", "beta"] + (["logf"] if args["logf"] is not None else [])
    fd = _fd_grads(orc, args, names)
    key = {"q": "dq", "k": "dk", "v": "dv", "w": "dw", "beta": "dbeta", "logf": "dlogf"}
    errs = {n: float(np.abs(g[key[n]] - fd[n]).max()) for n in names}
    return all(e < 1e-7 for e in errs.values()), errs


@pytest.mark.parametrize("gate", [False, True])
def test_bwd_matches_finite_differences(gate):
    ok, errs = _fd_matches(oracle.default(), _case(31, gate))
    assert ok, errs


def test_bwd_beta_zero_is_softmax_attention():
    S, L, d, dv = 2, 9, 4, 3
    q, k, v, w, _, _ = _rand_inputs(32, S, L, d, dv)
    beta = np.zeros((S, L))
    do = np.random.default_rng(33).standard_normal((S, L, dv))
    g = oracle.bwd(q, k, v, w, beta, None, SCALE, do)
    mask = np.tril(np.ones((L, L), dtype=bool))
    for s in range(S):
        A = np.where(mask, SCALE * q[s] @ k[s].T, -np.inf)
        P = np.exp(A - A.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = do[s] @ v[s].T
        dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
        np.testing.assert_allclose(g["dv"][s], P.T @ do[s], atol=1e-12)
        np.testing.assert_allclose(g["dq"][s], SCALE * dS @ k[s], atol=1e-12)
        np.testing.assert_allclose(g["dk"][s], SCALE * dS.T @ q[s], atol=1e-12)
        np.testing.assert_array_equal(g["dw"][s], 0.0)
        # d logit(i, j) / d beta_t = -scale (w_t . q_i)(w_t . k_j) for j < t <= i
        db = np.zeros(L)
        for t in range(L):
            for i in range(t, L):
                for j in range(t):
                    db[t] -= SCALE * dS[i, j] * (w[s, t] @ q[s, i]) * (w[s, t] @ k[s, j])
        np.testing.assert_allclose(g["dbeta"][s], db, atol=1e-12)


def test_bwd_first_position_has_no_gradient():
    a = _case(34, True, S=3, L=11, d=5, dv=4)
    g = oracle.bwd(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"], SCALE, a["do"])
    assert np.all(g["dw"][:, 0] == 0.0)
    assert np.all(g["dbeta"][:, 0] == 0.0)
    assert np.all(g["dlogf"][:, 0] == 0.0)
    # and the rest does get gradient
    assert np.abs(g["dw"][:, 1:]).min(axis=-1).max() > 0
    assert np.all(np.abs(g["dlogf"][:, 1:]) > 0)


# plausible mistakes in the reverse sweep; each must fail the finite differences
BWD_MUTANTS = {
    # the gradient carried past a transition without that transition
    "no_transition": ("g[e] - bs[j] * b * wj[e];", "g[e];"),
    # half of the rank-one derivative dropped (the (w . z) g term)
    "dw_half": ("(b * zj[e] + a * g[e])", "(b * zj[e])"),
    # wrong sign of the beta gradient
    "dbeta_sign": ("dbs[j] += -a * b;", "dbs[j] += a * b;"),
    # the softmax's row term dropped
    "softmax_row": ("(dot(dv, doi, vj) - D)", "dot(dv, doi, vj)"),
    # bias gradient given to the key's own position
    "dlogf_index": ("dfs[j + 1] += cum;", "dfs[j] += cum;"),
    # key gradient without the scale
    "dk_scale": ("+= scale * ds[j] * zj[e];", "+= ds[j] * zj[e];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_fails_pin(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "path_oracle.c")).read()
    old, new = BWD_MUTANTS[name]
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as tmp:
        csrc = os.path.join(tmp, "m.c")
        open(csrc, "w").write(src.replace(old, new))
        lib = oracle.build(os.path.join(tmp, "libm.so"), csrc)
        orc = oracle.Oracle(lib)
        caught = not _fd_matches(orc, _case(35, True, S=1, L=5, d=3, dv=2))[0]
    assert caught, name
