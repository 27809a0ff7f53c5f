"""fp64 CPU oracle for PaTH attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product library never does, and this package shares no
code with it.  The arithmetic lives in ``path_oracle.c`` (plain C, fp64,
OpenMP over independent query rows); this module only marshals numpy arrays.

What it computes (citations: the reading-notes page "PaTH Attention:通过累积
Householder 变换编码位置", sections 2.1, 2.5 and 2.8):

* ``fwd_rows``: for chosen query rows i, the PaTH(-FoX) attention output
  o_i and log-sum-exp lse_i, from logits
  scale * k_j^T H_{j+1}...H_i q_i + sum_{s=j+1..i} log f_s over j <= i.
* ``transported_keys``: the keys a decoding cache holds after position t,
  H_t...H_{j+1} k_j for j <= t.

* ``frontend``: the parameter branch that makes w_t (low-rank linear layer,
  width-3 causal short convolution, per-head L2 normalisation), beta_t =
  2 sigma(.) and log f_t = log sigma(.) from a layer input x_t (sections 2.1
  and 2.5; the reading of the unstated details is in path_oracle.c).

* ``bwd``: gradients of a scalar loss sum(do * o) with respect to q, k, v,
  w, beta and log f -- reverse-mode differentiation of the same walk (the
  pages give no backward formulas; finite differences of ``fwd_rows`` pin
  it).

Decode outputs need no function of their own: the output of the decode step
at position t is row t of ``fwd_rows`` on the prompt and decoded tokens
concatenated, which is what the pages' cache rewrite reproduces [s2.8].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "path_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
def build(out_path: str = _LIB_PATH, src_path: str = _SRC) -> str:
    """Compile path_oracle.c with gcc into a shared library (always recompiles)."""
    tmp = out_path + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall",
                    "-o", tmp, src_path, "-lm"], check=True)
    os.replace(tmp, out_path)
    return out_path


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Bindings to one compiled copy of path_oracle.c."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        lib.oracle_fwd_rows.argtypes = [ctypes.c_int] * 4 + [P] * 6 + [
            ctypes.c_double, ctypes.c_int, P, P, P]
        lib.oracle_fwd_rows.restype = ctypes.c_int
        lib.oracle_transported_keys.argtypes = [ctypes.c_int] * 3 + [P] * 3 + [
            ctypes.c_int, P]
        lib.oracle_transported_keys.restype = ctypes.c_int
        lib.oracle_frontend.argtypes = [ctypes.c_int] * 6 + [P] * 11
        lib.oracle_frontend.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [ctypes.c_int] * 4 + [P] * 6 + [ctypes.c_double] + [P] * 7
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self._lib = lib

    def frontend(self, x, Wd, Wu, kc, ub, bb, uf=None, bf=None, H=None, d=None):
        """Parameter front-end in fp64: (w [N,H,L,d], beta [N,H,L], logf [N,H,L] or None).

        x [N, L, Dm]; Wd [R, Dm]; Wu [H*d, R]; kc [H*d, 3]; ub, uf [H, Dm]; bb, bf [H].
        """
        x, Wd, Wu, kc, ub, bb = (_f64(a) for a in (x, Wd, Wu, kc, ub, bb))
        N, L, Dm = x.shape
        R = Wd.shape[0]
        H = ub.shape[0] if H is None else H
        d = Wu.shape[0] // H if d is None else d
        assert Wd.shape == (R, Dm) and Wu.shape == (H * d, R) and kc.shape == (H * d, 3)
        assert ub.shape == (H, Dm) and bb.shape == (H,)
        gate = uf is not None
        if gate:
            uf, bf = _f64(uf), _f64(bf)
            assert uf.shape == (H, Dm) and bf.shape == (H,)
        w = np.zeros((N, H, L, d))
        beta = np.zeros((N, H, L))
        logf = np.zeros((N, H, L)) if gate else None
        rc = self._lib.oracle_frontend(N, L, Dm, R, H, d, _ptr(x), _ptr(Wd), _ptr(Wu), _ptr(kc),
                                       _ptr(ub), _ptr(bb), _ptr(uf) if gate else None,
                                       _ptr(bf) if gate else None, _ptr(w), _ptr(beta),
                                       _ptr(logf) if gate else None)
        if rc != 0:
            raise RuntimeError("oracle_frontend failed")
        return w, beta, logf

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self._lib.oracle_set_num_threads(int(n))

    def fwd_rows(self, q, k, v, w, beta, logf=None, scale=1.0, rows=None):
        """PaTH(-FoX) attention for selected rows of S slices, in fp64.

        q, k, w: [S, L, d]; v: [S, L, dv]; beta, logf: [S, L] (logf None: PaTH).
        rows: None (all rows), a 1-D list used for every slice, or [S, nrows].
        Returns (o [S, nrows, dv], lse [S, nrows]) as float64 arrays.
        """
        q, k, v, w, beta = (_f64(x) for x in (q, k, v, w, beta))
        S, L, d = q.shape
        dv = v.shape[2]
        assert k.shape == (S, L, d) and w.shape == (S, L, d)
        assert v.shape[:2] == (S, L) and beta.shape == (S, L)
        if logf is not None:
            logf = _f64(logf)
            assert logf.shape == (S, L)
        if rows is None:
            rows = np.arange(L)
        rows = np.asarray(rows, dtype=np.int32)
        if rows.ndim == 1:
            rows = np.broadcast_to(rows, (S, rows.shape[0]))
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        assert rows.shape[0] == S
        nrows = rows.shape[1]
        o = np.empty((S, nrows, dv), dtype=np.float64)
        lse = np.empty((S, nrows), dtype=np.float64)
        rc = self._lib.oracle_fwd_rows(
            S, L, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
            _ptr(logf) if logf is not None else None, float(scale), nrows,
            _ptr(rows), _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("row index out of range")
        return o, lse

    def bwd(self, q, k, v, w, beta, logf=None, scale=1.0, do=None):
        """Gradients of sum(do * o) through PaTH(-FoX) attention, in fp64.

        Shapes as fwd_rows; do: [S, L, dv].  Returns a dict with dq, dk, dw
        [S, L, d], dv [S, L, dv], dbeta [S, L] and dlogf [S, L] (None without
        a gate).
        """
        q, k, v, w, beta, do = (_f64(x) for x in (q, k, v, w, beta, do))
        S, L, d = q.shape
        dv = v.shape[2]
        assert k.shape == (S, L, d) and w.shape == (S, L, d) and do.shape == (S, L, dv)
        assert v.shape[:2] == (S, L) and beta.shape == (S, L)
        if logf is not None:
            logf = _f64(logf)
            assert logf.shape == (S, L)
        out = dict(dq=np.empty((S, L, d)), dk=np.empty((S, L, d)), dv=np.empty((S, L, dv)),
                   dw=np.empty((S, L, d)), dbeta=np.empty((S, L)),
                   dlogf=np.empty((S, L)) if logf is not None else None)
        self._lib.oracle_bwd(
            S, L, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
            _ptr(logf) if logf is not None else None, float(scale), _ptr(do),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dw"]),
            _ptr(out["dbeta"]), _ptr(out["dlogf"]) if logf is not None else None)
        return out

    def transported_keys(self, k, w, beta, t):
        """Keys after position t is processed: H_t...H_{j+1} k_j, j in [0, t].

        k, w: [S, L, d]; beta: [S, L]. Returns [S, t+1, d] float64.
        """
        k, w, beta = _f64(k), _f64(w), _f64(beta)
        S, L, d = k.shape
        out = np.empty((S, t + 1, d), dtype=np.float64)
        rc = self._lib.oracle_transported_keys(S, L, d, _ptr(k), _ptr(w),
                                               _ptr(beta), int(t), _ptr(out))
        if rc != 0:
            raise ValueError("t out of range")
        return out


_default = None


def default() -> Oracle:
    """The oracle built in-tree (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def fwd_rows(*args, **kwargs):
    return default().fwd_rows(*args, **kwargs)


def transported_keys(*args, **kwargs):
    return default().transported_keys(*args, **kwargs)


def frontend(*args, **kwargs):
    return default().frontend(*args, **kwargs)


def bwd(*args, **kwargs):
    return default().bwd(*args, **kwargs)
