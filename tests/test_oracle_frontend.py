"""Pins of the oracle's parameter front-end (w_t, beta_t, log f_t from x_t).

The front-end is the branch the reading-notes page describes in its
sections 2.1 and 2.5: a low-rank linear layer, a width-3 short convolution
and L2 normalisation for w_t; beta_t = 2 sigma(.); log f_t = log sigma(.).
Every check below is fixed by something other than the oracle itself:
closed forms of sigma at chosen points, one-hot (selection) weights that
reduce the projections to indexing, shifts of the causal convolution,
normalisation invariants.  Planted mistakes in a copy of the oracle must
fail at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "path_oracle.c")


def _rand(seed, N=2, L=9, Dm=12, R=4, H=3, d=5):
    g = np.random.default_rng(seed)
    return dict(x=g.normal(size=(N, L, Dm)), Wd=g.normal(size=(R, Dm)),
                Wu=g.normal(size=(H * d, R)), kc=g.normal(size=(H * d, 3)),
                ub=g.normal(size=(H, Dm)), bb=g.normal(size=H),
                uf=g.normal(size=(H, Dm)), bf=g.normal(size=H))


def _selection(seed, taps, N=1, L=8, Dm=10, H=2, d=4):
    """One-hot weights: r_t[ch] = x_t[src[ch]], so every intermediate is known."""
    g = np.random.default_rng(seed)
    R = 6
    sel_d = g.choice(Dm, size=R, replace=False)        # p_t[j] = x_t[sel_d[j]]
    sel_u = g.integers(0, R, size=H * d)                # r_t[ch] = p_t[sel_u[ch]]
    Wd = np.zeros((R, Dm)); Wd[np.arange(R), sel_d] = 1.0
    Wu = np.zeros((H * d, R)); Wu[np.arange(H * d), sel_u] = 1.0
    kc = np.tile(np.asarray(taps, float), (H * d, 1))
    x = g.normal(size=(N, L, Dm))
    src = sel_d[sel_u]
    p = dict(x=x, Wd=Wd, Wu=Wu, kc=kc, ub=np.zeros((H, Dm)), bb=np.zeros(H))
    return p, src, H, d


def _expected_selection(x, src, taps, H, d):
    N, L, _ = x.shape
    r = x[:, :, src]                                    # [N, L, H*d]
    c = np.zeros_like(r)
    for tau, a in enumerate(taps):
        if a != 0.0:
            c[:, tau:, :] += a * r[:, :L - tau, :] if tau else a * r
    c = c.reshape(N, L, H, d).transpose(0, 2, 1, 3)
    n = np.sqrt((c * c).sum(-1, keepdims=True))
    return np.where(n > 0, c / np.where(n > 0, n, 1.0), 0.0)


def _check_all(orc):
    """Every pin, as booleans (shared with the mutant tests)."""
    res = {}
    # beta = 2 sigma(b) at b = 0, +-log 3: 1, 3/2, 1/2
    p = _rand(1, N=1, L=3, H=3)
    p["ub"][:] = 0.0
    p["bb"] = np.array([0.0, math.log(3.0), -math.log(3.0)])
    p["uf"][:] = 0.0
    p["bf"] = np.array([0.0, math.log(3.0), -60.0])
    w, beta, logf = orc.frontend(**p)
    res["beta"] = np.allclose(beta[0, :, 0], [1.0, 1.5, 0.5], rtol=0, atol=1e-15)
    # log sigma(0) = -ln 2, log sigma(ln 3) = ln(3/4), log sigma(-60) = -60 - ln(1 + e^-60)
    res["logf"] = (abs(logf[0, 0, 0] + math.log(2.0)) < 1e-15 and
                   abs(logf[0, 1, 0] - math.log(0.75)) < 1e-15 and
                   abs(logf[0, 2, 0] + 60.0) < 1e-12)
    # selection weights reduce the projections to indexing; taps act as shifts
    ok = True
    for taps in ((1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.5, -2.0, 1.5)):
        q, src, H, d = _selection(7, taps)
        w, _, _ = orc.frontend(**q)
        ok &= np.abs(w - _expected_selection(q["x"], src, taps, H, d)).max() < 1e-14
    res["selection"] = bool(ok)
    # unit norm, invariance to a positive scale of Wu, sign flip for a negative one
    p = _rand(3)
    w, beta, logf = orc.frontend(**p)
    q = dict(p); q["Wu"] = 3.7 * p["Wu"]
    w2, _, _ = orc.frontend(**q)
    q["Wu"] = -2.0 * p["Wu"]
    w3, _, _ = orc.frontend(**q)
    res["norm"] = bool(np.abs(np.linalg.norm(w, axis=-1) - 1.0).max() < 1e-13
                       and np.abs(w2 - w).max() < 1e-13 and np.abs(w3 + w).max() < 1e-13)
    # beta in (0, 2) and log f < 0 on random inputs
    res["ranges"] = bool((beta > 0).all() and (beta < 2).all() and (logf < 0).all())
    return res


def test_frontend_pins():
    res = _check_all(oracle.default())
    assert all(res.values()), res


def test_frontend_without_gate():
    p = _rand(5)
    w, beta, logf = oracle.frontend(**p)
    q = dict(p); q.pop("uf"); q.pop("bf")
    w2, beta2, logf2 = oracle.frontend(**q)
    assert logf2 is None
    assert np.array_equal(w, w2) and np.array_equal(beta, beta2)


def test_zero_input_gives_zero_w():
    p = _rand(6)
    p["x"][:] = 0.0
    w, beta, _ = oracle.frontend(**p)
    assert not w.any()
    assert np.allclose(beta, 2.0 / (1.0 + np.exp(-p["bb"]))[None, :, None], rtol=0, atol=1e-15)


FE_MUTANTS = {
    "beta_factor": ("beta[o] = 2.0 / (1.0 + exp(-zb));", "beta[o] = 1.0 / (1.0 + exp(-zb));"),
    "logsig_sign": ("return z >= 0.0 ? -log1p(exp(-z))", "return z >= 0.0 ? log1p(exp(-z))"),
    "no_norm": ("const double inv = nrm2 > 0.0 ? 1.0 / sqrt(nrm2) : 0.0;",
                "const double inv = nrm2 > 0.0 ? 1.0 : 0.0;"),
    "taps_reversed": ("s += kc[(size_t)ch * 3 + tau]", "s += kc[(size_t)ch * 3 + (2 - tau)]"),
    "anticausal": ("if (t - tau >= 0) s += kc[(size_t)ch * 3 + tau] * r[(size_t)(t - tau) * C + ch];",
                   "if (t + tau < L) s += kc[(size_t)ch * 3 + tau] * r[(size_t)(t + tau) * C + ch];"),
    "wu_row": ("dot(R, Wu + (size_t)ch * R, p", "dot(R, Wu + (size_t)(ch % R) * R, p"),
}


@pytest.mark.parametrize("name", sorted(FE_MUTANTS))
def test_frontend_mutant_is_caught(name, tmp_path):
    old, new = FE_MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = oracle.build(str(tmp_path / "libmutant.so"), str(mutated))
    res = _check_all(oracle.Oracle(lib))
    assert not all(res.values()), f"mutant {name} survived the pins"
