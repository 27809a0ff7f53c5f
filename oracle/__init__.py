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
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self._lib = lib

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

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


def fwd_rows(*args, **kwargs):
    return default().fwd_rows(*args, **kwargs)


def transported_keys(*args, **kwargs):
    return default().transported_keys(*args, **kwargs)
