"""Plant plausible mistakes in a copy of the oracle and check that a pin fails.

Each mutant is a textual edit of path_oracle.c compiled into a temporary
library on the CPU.  The pins used here are the brute-force product check and
the forget-gate reduction; if a mutant passed all of them the pins would be
too weak to trust the oracle.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _bruteforce_logits, _rand_inputs, _softmax_out

SRC = os.path.join(os.path.dirname(oracle.__file__), "path_oracle.c")

MUTANTS = {
    # score read after the transition: H_j enters key j's path (wrong endpoint)
    "endpoint_shift": (
        "        scores[j] = scale * dot(d, k + (size_t)j * d, z) + bias;\n"
        "        apply_transition(d, w + (size_t)j * d, beta[j], z);   /* z <- H_j z */\n",
        "        apply_transition(d, w + (size_t)j * d, beta[j], z);   /* z <- H_j z */\n"
        "        scores[j] = scale * dot(d, k + (size_t)j * d, z) + bias;\n"),
    # wrong sign of the rank-one correction
    "sign": ("z[e] -= beta * wz * w[e];", "z[e] += beta * wz * w[e];"),
    # dropped beta
    "dropped_beta": ("z[e] -= beta * wz * w[e];", "z[e] -= wz * w[e];"),
    # bias accumulated one position early (includes log f_j for key j)
    "bias_index": ("        if (logf) bias += logf[j];\n", ""),
    # scale dropped
    "no_scale": ("scores[j] = scale * dot(", "scores[j] = dot("),
    # transition taken from the wrong position (off by one)
    "w_index": ("apply_transition(d, w + (size_t)j * d, beta[j], z);",
                "apply_transition(d, w + (size_t)(j > 0 ? j - 1 : 0) * d, beta[j], z);"),
}


def _pins_pass(orc):
    ok = True
    for fox in (False, True):
        q, k, v, w, beta, logf = _rand_inputs(21, 2, 8, 4)
        lf = logf if fox else None
        if fox:   # the gate-bias pin needs an already-correct bias position
            lf = lf.copy()
            lf[:, :] = np.where(np.arange(8) % 2 == 0, -0.5, -0.1)
        o, lse = orc.fwd_rows(q, k, v, w, beta, lf, 0.7)
        for s in range(2):
            A = _bruteforce_logits(q[s], k[s], w[s], beta[s], None if lf is None else lf[s], 0.7)
            o_ref, lse_ref = _softmax_out(A, v[s])
            ok &= np.abs(o[s] - o_ref).max() < 1e-10 and np.abs(lse[s] - lse_ref).max() < 1e-10
    if orc.transported_keys is not None:
        q, k, v, w, beta, _ = _rand_inputs(22, 1, 6, 3)
        kt = orc.transported_keys(k, w, beta, 5)
        M = np.eye(3)
        for s in range(1, 6):
            M = (np.eye(3) - beta[0, s] * np.outer(w[0, s], w[0, s])) @ M
        ok &= np.abs(kt[0, 0] - M @ k[0, 0]).max() < 1e-10
    return bool(ok)


def test_unmutated_copy_passes(tmp_path):
    lib = oracle.build(str(tmp_path / "liboracle_copy.so"), SRC)
    assert _pins_pass(oracle.Oracle(lib))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = oracle.build(str(tmp_path / "libmutant.so"), str(mutated))
    assert not _pins_pass(oracle.Oracle(lib)), f"mutant {name} survived the pins"
