"""libpath_attn: PaTH attention prefill and decode for AMD Instinct MI355X.

Thin ctypes binding over the C ABI in include/path_attn.h.  It only marshals
arguments: torch tensors supply device memory and the current stream; every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if libpath_attn.so is missing or a call fails, an exception is
raised.

The operation (reading-notes page "PaTH Attention:通过累积 Householder
变换编码位置", sections 2.1 and 2.5): with H_t = I - beta_t w_t w_t^T,
    logit(i, j) = scale * k_j^T H_{j+1}...H_i q_i + sum_{s=j+1..i} log f_s,
for j <= i, then a causal softmax and the value sum; lse is the natural-log
log-sum-exp of each row's logits.  Decoding (section 2.8) keeps keys already
rewritten by every later transition, so a plain softmax over the cache gives
the same scores.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpath_attn.so")

PATH_F32, PATH_BF16 = 0, 1
_STATUS = ["ok", "null pointer", "bad shape", "bad dtype", "unsupported",
           "misaligned pointer", "workspace too small", "cache capacity exceeded",
           "kernel launch failed"]


class PathAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        self.status = status
        name = _STATUS[status] if 0 <= status < len(_STATUS) else str(status)
        super().__init__(f"libpath_attn: {name} ({status}): {msg}")


class _Desc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("L", ctypes.c_int),
                ("d", ctypes.c_int), ("dtype", ctypes.c_int), ("scale", ctypes.c_float),
                ("block", ctypes.c_int)]


class _ParamDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("L", ctypes.c_int), ("Dm", ctypes.c_int),
                ("R", ctypes.c_int), ("H", ctypes.c_int), ("d", ctypes.c_int),
                ("dtype", ctypes.c_int)]


class _Cache(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int), ("k_dtype", ctypes.c_int),
                ("kcache", ctypes.c_void_p), ("vcache", ctypes.c_void_p),
                ("gcache", ctypes.c_void_p)]


class _PagedCache(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int), ("page_size", ctypes.c_int),
                ("k_dtype", ctypes.c_int), ("kpages", ctypes.c_void_p),
                ("vpages", ctypes.c_void_p), ("gpages", ctypes.c_void_p)]


_lib = None

EXPORTS = ["path_abi_version", "path_status_str", "path_last_error",
           "path_attn_fwd_workspace", "path_attn_fwd", "path_kv_update",
           "path_kv_append", "path_decode_workspace", "path_decode",
           "path_decode_step", "path_causal_attn_fwd", "path_attn_fwd_timed",
           "path_param_workspace", "path_param_fwd", "path_attn_bwd_workspace",
           "path_attn_bwd", "path_paged_decode_workspace", "path_paged_decode_step",
           "path_paged_import", "path_decode_step_noalloc", "path_decode_step_noalloc_limit"]


def load_library(path: str = LIB_PATH):
    """Load libpath_attn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libpath_attn.so not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    DP, CP = ctypes.POINTER(_Desc), ctypes.POINTER(_Cache)
    sig = {
        "path_abi_version": ([], I),
        "path_status_str": ([I], ctypes.c_char_p),
        "path_last_error": ([], ctypes.c_char_p),
        "path_attn_fwd_workspace": ([DP, I], S),
        "path_attn_fwd": ([DP, P, P, P, P, P, P, P, P, CP, P, S, P], I),
        "path_kv_update": ([DP, CP, I, P, P, P], I),
        "path_kv_append": ([DP, CP, I, P, P, P, P], I),
        "path_decode_workspace": ([DP, I], S),
        "path_decode": ([DP, CP, I, P, P, P, P, S, P], I),
        "path_decode_step": ([DP, CP, I, P, P, P, P, P, P, P, P, P, S, P], I),
        "path_causal_attn_fwd": ([DP, P, P, P, P, P, P], I),
        "path_attn_fwd_timed": ([DP, P, P, P, P, P, P, P, P, CP, P, S, P, P], I),
        "path_param_workspace": ([ctypes.POINTER(_ParamDesc), I], S),
        "path_param_fwd": ([ctypes.POINTER(_ParamDesc)] + [P] * 12 + [S, P], I),
        "path_attn_bwd_workspace": ([DP], S),
        "path_attn_bwd": ([DP] + [P] * 16 + [S, P], I),
        "path_paged_decode_workspace": ([DP, I], S),
        "path_paged_decode_step": ([DP, ctypes.POINTER(_PagedCache), P, I, P, I] + [P] * 9
                                   + [S, P], I),
        "path_paged_import": ([DP, CP, ctypes.POINTER(_PagedCache), P, I, P, I, P], I),
        "path_decode_step_noalloc": ([DP, CP, I, P, P, P, P, P, P, P, P, P], I),
        "path_decode_step_noalloc_limit": ([], S),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PathAttnError(status, _lib.path_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return PATH_F32
    if t == torch.bfloat16:
        return PATH_BF16
    raise PathAttnError(3, f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dev, shape=None, dtype=None):
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _workspace(workspace, nbytes: int, dev):
    """The caller's workspace if it is a large enough uint8 tensor on dev, else a new one."""
    if workspace is not None:
        _need(workspace, "workspace", dev, None, torch.uint8)
        if workspace.numel() >= nbytes:
            return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)


_OPTIONAL = ("lse", "lse_t")  # the C calls accept NULL for these outputs


def _outs(out, dev, specs):
    """Validate caller-provided output tensors against (name, shape, dtype)
    specs; shape None means the output must be absent."""
    if len(out) != len(specs):
        raise ValueError(f"out must hold {len(specs)} tensors, got {len(out)}")
    for t, (name, shape, dtype) in zip(out, specs):
        if t is None:
            if shape is not None and name not in _OPTIONAL:
                raise ValueError(f"out: {name} is required")
            continue
        if shape is None:
            raise ValueError(f"out: {name} must be None here")
        _need(t, name, dev, shape, dtype)
    return out


def _desc(N, H, L, d, dtype, scale, block=0):
    return _Desc(N, H, L, d, _dtype_code(dtype), float(scale), int(block))


def fwd_workspace_bytes(N, H, L, d, dtype, with_cache=False, block=0) -> int:
    lib = load_library()
    return int(lib.path_attn_fwd_workspace(ctypes.byref(_desc(N, H, L, d, dtype, 1.0, block)),
                                           int(bool(with_cache))))


class Cache:
    """Decode cache: kcache/vcache [N,H,cap,d], gcache [N,H,cap] (or None).

    kcache holds every key rewritten by all transitions after it; gcache holds
    inclusive prefix sums of log f when the forget gate is used.
    """

    def __init__(self, N, H, cap, d, dtype=torch.bfloat16, k_dtype=None,
                 gate=True, device="cuda"):
        self.N, self.H, self.cap, self.d = N, H, cap, d
        self.dtype = dtype
        self.k_dtype = dtype if k_dtype is None else k_dtype
        self.kcache = torch.zeros(N, H, cap, d, dtype=self.k_dtype, device=device)
        self.vcache = torch.zeros(N, H, cap, d, dtype=dtype, device=device)
        self.gcache = torch.zeros(N, H, cap, dtype=torch.float32, device=device) if gate else None
        self.device = self.kcache.device

    def _c(self):
        return _Cache(self.cap, _dtype_code(self.k_dtype), self.kcache.data_ptr(),
                      self.vcache.data_ptr(),
                      self.gcache.data_ptr() if self.gcache is not None else None)


def fwd(q, k, v, w, beta, logf=None, scale=None, cache: Cache | None = None,
        block=0, workspace: torch.Tensor | None = None, out=None, events=None):
    """Prefill forward.  q,k,v,w [N,H,L,d] (fp32 or bf16); beta, logf [N,H,L] fp32.

    Returns (o [N,H,L,d], lse [N,H,L] fp32).  If cache is given, it is filled
    with the prompt's keys aligned to the last position, values and log-f
    prefix sums.
    """
    lib = load_library()
    N, H, L, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("w", w)):
        _need(t, name, dev, (N, H, L, d), q.dtype)
    _need(beta, "beta", dev, (N, H, L), torch.float32)
    if logf is not None:
        _need(logf, "logf", dev, (N, H, L), torch.float32)
    if cache is not None:
        if (cache.N, cache.H, cache.d) != (N, H, d) or cache.dtype != q.dtype:
            raise ValueError(f"cache is [{cache.N},{cache.H},cap,{cache.d}] {cache.dtype}, "
                             f"inputs are [{N},{H},{L},{d}] {q.dtype}")
        if cache.device != dev:
            raise ValueError(f"cache must be on {dev}")
    scale = d ** -0.5 if scale is None else scale
    desc = _desc(N, H, L, d, q.dtype, scale, block)
    nbytes = int(lib.path_attn_fwd_workspace(ctypes.byref(desc), int(cache is not None)))
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(N, H, L, dtype=torch.float32, device=dev)
    else:
        o, lse = _outs(out, dev, [("o", (N, H, L, d), q.dtype), ("lse", (N, H, L), torch.float32)])
    cc = cache._c() if cache is not None else None
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf),
            _ptr(o), _ptr(lse), ctypes.byref(cc) if cc is not None else None,
            _ptr(workspace), workspace.numel(), _stream(dev))
    if events is None:
        _check(lib.path_attn_fwd(*args))
    else:
        # events: four torch.cuda.Event(enable_timing=True), recorded by the library
        evs = (ctypes.c_void_p * 4)(*[e.cuda_event for e in _init_events(events, dev)])
        _check(lib.path_attn_fwd_timed(*args, evs))
    return o, lse


def bwd_workspace_bytes(N, H, L, d, dtype, block=0) -> int:
    lib = load_library()
    return int(lib.path_attn_bwd_workspace(ctypes.byref(_desc(N, H, L, d, dtype, 1.0, block))))


def bwd(q, k, v, w, beta, logf, o, lse, do, scale=None, workspace=None, out=None):
    """Backward pass: gradients of a loss through fwd(), given do = dL/do.

    q, k, v, w, o, do [N,H,L,d] (fp32 or bf16); beta, logf, lse [N,H,L] fp32
    (logf None: plain PaTH).  Returns (dq, dk, dv, dw, dbeta, dlogf) with
    dlogf None without a gate.
    """
    lib = load_library()
    N, H, L, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("w", w), ("o", o), ("do", do)):
        _need(t, name, dev, (N, H, L, d), q.dtype)
    for name, t in (("beta", beta), ("lse", lse)):
        _need(t, name, dev, (N, H, L), torch.float32)
    if logf is not None:
        _need(logf, "logf", dev, (N, H, L), torch.float32)
    scale = d ** -0.5 if scale is None else scale
    desc = _desc(N, H, L, d, q.dtype, scale)
    nbytes = int(lib.path_attn_bwd_workspace(ctypes.byref(desc)))
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        dq, dk, dv, dw = (torch.empty_like(q) for _ in range(4))
        dbeta = torch.empty(N, H, L, dtype=torch.float32, device=dev)
        dlogf = torch.empty(N, H, L, dtype=torch.float32, device=dev) if logf is not None else None
    else:
        full, row = (N, H, L, d), (N, H, L)
        dq, dk, dv, dw, dbeta, dlogf = _outs(out, dev, [
            ("dq", full, q.dtype), ("dk", full, q.dtype), ("dv", full, q.dtype),
            ("dw", full, q.dtype), ("dbeta", row, torch.float32),
            ("dlogf", row if logf is not None else None, torch.float32)])
    _check(lib.path_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
                             _ptr(logf), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dw), _ptr(dbeta), _ptr(dlogf), _ptr(workspace),
                             workspace.numel(), _stream(dev)))
    return dq, dk, dv, dw, dbeta, dlogf


def _init_events(events, dev):
    """torch creates the underlying hipEvent lazily; force it into existence."""
    for e in events:
        if e.cuda_event == 0:
            e.record(torch.cuda.current_stream(dev))
    return events


def _token_outs(N, H, d, dtype, dev, q_t, out):
    """(o_t, lse_t) for one decode position: new tensors, or the caller's, validated."""
    if out is None:
        return (torch.empty_like(q_t),
                torch.empty(N, H, dtype=torch.float32, device=dev))
    return _outs(out, dev, [("o_t", (N, H, d), dtype), ("lse_t", (N, H), torch.float32)])


def _cache_desc(cache: Cache, scale):
    return _desc(cache.N, cache.H, 1, cache.d, cache.dtype, scale)


def kv_update(cache: Cache, n: int, w_t, beta_t):
    """k_j <- k_j - beta_t (w_t . k_j) w_t for slots j < n (in place)."""
    lib = load_library()
    _need(w_t, "w_t", cache.device, (cache.N, cache.H, cache.d), cache.dtype)
    _need(beta_t, "beta_t", cache.device, (cache.N, cache.H), torch.float32)
    desc = _cache_desc(cache, 1.0)
    cc = cache._c()
    _check(lib.path_kv_update(ctypes.byref(desc), ctypes.byref(cc), int(n), _ptr(w_t),
                              _ptr(beta_t), _stream(cache.device)))


def kv_append(cache: Cache, n: int, k_t, v_t, logf_t=None):
    """Write token n: key (unrewritten), value and log-f prefix."""
    lib = load_library()
    for name, t in (("k_t", k_t), ("v_t", v_t)):
        _need(t, name, cache.device, (cache.N, cache.H, cache.d), cache.dtype)
    if logf_t is not None:
        _need(logf_t, "logf_t", cache.device, (cache.N, cache.H), torch.float32)
    desc = _cache_desc(cache, 1.0)
    cc = cache._c()
    _check(lib.path_kv_append(ctypes.byref(desc), ctypes.byref(cc), int(n), _ptr(k_t),
                              _ptr(v_t), _ptr(logf_t), _stream(cache.device)))


def decode_workspace_bytes(cache: Cache, n_keys: int) -> int:
    lib = load_library()
    return int(lib.path_decode_workspace(ctypes.byref(_cache_desc(cache, 1.0)), int(n_keys)))


def decode(cache: Cache, n_keys: int, q_t, scale=None, workspace=None, out=None):
    """Attend q_t [N,H,d] over cache slots [0, n_keys). Returns (o_t, lse_t)."""
    lib = load_library()
    _need(q_t, "q_t", cache.device, (cache.N, cache.H, cache.d), cache.dtype)
    scale = cache.d ** -0.5 if scale is None else scale
    desc = _cache_desc(cache, scale)
    nbytes = decode_workspace_bytes(cache, n_keys)
    workspace = _workspace(workspace, nbytes, cache.device)
    o, lse = _token_outs(cache.N, cache.H, cache.d, cache.dtype, cache.device, q_t, out)
    cc = cache._c()
    _check(lib.path_decode(ctypes.byref(desc), ctypes.byref(cc), int(n_keys), _ptr(q_t),
                           _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
                           _stream(cache.device)))
    return o, lse


def decode_step(cache: Cache, n: int, q_t, k_t, v_t, w_t, beta_t, logf_t=None,
                scale=None, workspace=None, out=None):
    """Fused step at position n: rewrite slots < n, append token n, attend."""
    lib = load_library()
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _need(t, name, cache.device, (cache.N, cache.H, cache.d), cache.dtype)
    _need(beta_t, "beta_t", cache.device, (cache.N, cache.H), torch.float32)
    if logf_t is not None:
        _need(logf_t, "logf_t", cache.device, (cache.N, cache.H), torch.float32)
    scale = cache.d ** -0.5 if scale is None else scale
    desc = _cache_desc(cache, scale)
    nbytes = decode_workspace_bytes(cache, n + 1)
    workspace = _workspace(workspace, nbytes, cache.device)
    o, lse = _token_outs(cache.N, cache.H, cache.d, cache.dtype, cache.device, q_t, out)
    cc = cache._c()
    _check(lib.path_decode_step(ctypes.byref(desc), ctypes.byref(cc), int(n), _ptr(q_t),
                                _ptr(k_t), _ptr(v_t), _ptr(w_t), _ptr(beta_t), _ptr(logf_t),
                                _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
                                _stream(cache.device)))
    return o, lse


def decode_step_noalloc_limit() -> int:
    """Bytes of the library's device-resident scratch that decode_step_noalloc uses."""
    return int(load_library().path_decode_step_noalloc_limit())


def decode_step_noalloc(cache: Cache, n: int, q_t, k_t, v_t, w_t, beta_t, logf_t=None,
                        scale=None, out=None):
    """decode_step without a workspace: the split-K partial states go to a
    scratch array the library keeps in device memory (one per GPU, shared by
    every call on it, so overlapping calls on one GPU race).  For callers that
    cannot allocate: pass `out` to make the call allocate nothing at all."""
    lib = load_library()
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _need(t, name, cache.device, (cache.N, cache.H, cache.d), cache.dtype)
    _need(beta_t, "beta_t", cache.device, (cache.N, cache.H), torch.float32)
    if logf_t is not None:
        _need(logf_t, "logf_t", cache.device, (cache.N, cache.H), torch.float32)
    scale = cache.d ** -0.5 if scale is None else scale
    desc = _cache_desc(cache, scale)
    o, lse = _token_outs(cache.N, cache.H, cache.d, cache.dtype, cache.device, q_t, out)
    cc = cache._c()
    _check(lib.path_decode_step_noalloc(ctypes.byref(desc), ctypes.byref(cc), int(n), _ptr(q_t),
                                        _ptr(k_t), _ptr(v_t), _ptr(w_t), _ptr(beta_t),
                                        _ptr(logf_t), _ptr(o), _ptr(lse), _stream(cache.device)))
    return o, lse


class PagedCache:
    """Paged decode cache for a batch of sequences: kpages/vpages
    [num_pages, H, page_size, d], gpages [num_pages, H, page_size] (or None).

    A sequence's slots [i*page_size, (i+1)*page_size) live in the page its
    table row names at entry i; slots hold rewritten keys as in Cache.
    """

    def __init__(self, num_pages, page_size, H, d, dtype=torch.bfloat16, k_dtype=None,
                 gate=True, device="cuda"):
        self.num_pages, self.page_size, self.H, self.d = num_pages, page_size, H, d
        self.dtype = dtype
        self.k_dtype = dtype if k_dtype is None else k_dtype
        self.kpages = torch.zeros(num_pages, H, page_size, d, dtype=self.k_dtype, device=device)
        self.vpages = torch.zeros(num_pages, H, page_size, d, dtype=dtype, device=device)
        self.gpages = (torch.zeros(num_pages, H, page_size, dtype=torch.float32, device=device)
                       if gate else None)
        self.device = self.kpages.device

    def _c(self):
        return _PagedCache(self.num_pages, self.page_size, _dtype_code(self.k_dtype),
                           self.kpages.data_ptr(), self.vpages.data_ptr(),
                           self.gpages.data_ptr() if self.gpages is not None else None)


def _paged_tables(cache: PagedCache, page_table, seq_lens, max_keys):
    S = seq_lens.shape[0]
    _need(seq_lens, "seq_lens", cache.device, (S,), torch.int32)
    if page_table.dim() != 2 or page_table.shape[0] != S:
        raise ValueError(f"page_table must be [S, table_stride], got {tuple(page_table.shape)}")
    _need(page_table, "page_table", cache.device, None, torch.int32)
    return S, page_table.shape[1]


def paged_decode_workspace_bytes(S, H, d, dtype, max_keys) -> int:
    lib = load_library()
    return int(lib.path_paged_decode_workspace(ctypes.byref(_desc(S, H, 1, d, dtype, 1.0)),
                                               int(max_keys)))


def paged_decode_step(cache: PagedCache, page_table, seq_lens, max_keys, q_t, k_t, v_t, w_t,
                      beta_t, logf_t=None, scale=None, workspace=None, out=None):
    """Fused step for a batch of S sequences at positions seq_lens (int32 [S],
    advanced by one): rewrite each sequence's cached keys, append its token,
    attend.  q_t, k_t, v_t, w_t [S,H,d]; beta_t, logf_t [S,H] fp32; page_table
    int32 [S, table_stride].  Returns (o_t [S,H,d], lse_t [S,H])."""
    lib = load_library()
    S, stride = _paged_tables(cache, page_table, seq_lens, max_keys)
    H, d = cache.H, cache.d
    for name, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("w_t", w_t)):
        _need(t, name, cache.device, (S, H, d), cache.dtype)
    _need(beta_t, "beta_t", cache.device, (S, H), torch.float32)
    if logf_t is not None:
        _need(logf_t, "logf_t", cache.device, (S, H), torch.float32)
    scale = d ** -0.5 if scale is None else scale
    desc = _desc(S, H, 1, d, cache.dtype, scale)
    nbytes = paged_decode_workspace_bytes(S, H, d, cache.dtype, max_keys)
    workspace = _workspace(workspace, nbytes, cache.device)
    o, lse = _token_outs(S, H, d, cache.dtype, cache.device, q_t, out)
    pc = cache._c()
    _check(lib.path_paged_decode_step(ctypes.byref(desc), ctypes.byref(pc), _ptr(page_table),
                                      int(stride), _ptr(seq_lens), int(max_keys), _ptr(q_t),
                                      _ptr(k_t), _ptr(v_t), _ptr(w_t), _ptr(beta_t),
                                      _ptr(logf_t), _ptr(o), _ptr(lse), _ptr(workspace),
                                      workspace.numel(), _stream(cache.device)))
    return o, lse


def paged_import(src: Cache, dst: PagedCache, page_table, seq_lens, max_keys):
    """Copy slots [0, seq_lens[s]) of each sequence of a contiguous cache into
    its pages (src.N = S sequences)."""
    lib = load_library()
    S, stride = _paged_tables(dst, page_table, seq_lens, max_keys)
    if src.N != S or src.H != dst.H or src.d != dst.d:
        raise ValueError("source cache and paged cache shapes differ")
    if src.dtype != dst.dtype or src.k_dtype != dst.k_dtype:
        raise ValueError(f"source cache ({src.dtype}, keys {src.k_dtype}) and paged cache "
                         f"({dst.dtype}, keys {dst.k_dtype}) dtypes differ")
    if (src.gcache is None) != (dst.gpages is None):
        raise ValueError("source cache and paged cache must both have a gate prefix or neither")
    if src.device != dst.device:
        raise ValueError("source cache and paged cache are on different devices")
    desc = _desc(S, dst.H, 1, dst.d, dst.dtype, 1.0)
    sc, pc = src._c(), dst._c()
    _check(lib.path_paged_import(ctypes.byref(desc), ctypes.byref(sc), ctypes.byref(pc),
                                 _ptr(page_table), int(stride), _ptr(seq_lens), int(max_keys),
                                 _stream(dst.device)))


def causal_attn(q, k, v, scale=None, out=None):
    """Plain causal softmax attention (the beta = 0 baseline kernel)."""
    lib = load_library()
    N, H, L, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.device, (N, H, L, d), q.dtype)
    scale = d ** -0.5 if scale is None else scale
    desc = _desc(N, H, L, d, q.dtype, scale)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(N, H, L, dtype=torch.float32, device=q.device)
    else:
        o, lse = _outs(out, q.device, [("o", (N, H, L, d), q.dtype),
                                       ("lse", (N, H, L), torch.float32)])
    _check(lib.path_causal_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    _ptr(lse), _stream(q.device)))
    return o, lse


def param_workspace_bytes(N, L, Dm, R, H, d, dtype, gate=True) -> int:
    lib = load_library()
    desc = _ParamDesc(N, L, Dm, R, H, d, _dtype_code(dtype))
    return int(lib.path_param_workspace(ctypes.byref(desc), 1 if gate else 0))


def param_fwd(x, Wd, Wu, kc, ub, bb, uf=None, bf=None, H=None, d=None, workspace=None,
              out=None):
    """Parameter front-end: (w [N,H,L,d], beta [N,H,L], logf [N,H,L] or None).

    x [N, L, Dm]; Wd [R, Dm]; Wu [H*d, R]; ub, uf [H, Dm] in x's dtype;
    kc [H*d, 3], bb, bf [H] float32.  uf and bf together enable the gate.
    """
    lib = load_library()
    N, L, Dm = x.shape
    R = Wd.shape[0]
    H = ub.shape[0] if H is None else H
    d = Wu.shape[0] // H if d is None else d
    dev = x.device
    _need(x, "x", dev, (N, L, Dm), x.dtype)
    _need(Wd, "Wd", dev, (R, Dm), x.dtype)
    _need(Wu, "Wu", dev, (H * d, R), x.dtype)
    _need(ub, "ub", dev, (H, Dm), x.dtype)
    _need(kc, "kc", dev, (H * d, 3), torch.float32)
    _need(bb, "bb", dev, (H,), torch.float32)
    gate = uf is not None
    if gate:
        _need(uf, "uf", dev, (H, Dm), x.dtype)
        _need(bf, "bf", dev, (H,), torch.float32)
    desc = _ParamDesc(N, L, Dm, R, H, d, _dtype_code(x.dtype))
    nbytes = int(lib.path_param_workspace(ctypes.byref(desc), 1 if gate else 0))
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        w = torch.empty(N, H, L, d, dtype=x.dtype, device=dev)
        beta = torch.empty(N, H, L, dtype=torch.float32, device=dev)
        logf = torch.empty(N, H, L, dtype=torch.float32, device=dev) if gate else None
    else:
        w, beta, logf = _outs(out, dev, [("w", (N, H, L, d), x.dtype),
                                         ("beta", (N, H, L), torch.float32),
                                         ("logf", (N, H, L) if gate else None, torch.float32)])
    _check(lib.path_param_fwd(ctypes.byref(desc), _ptr(x), _ptr(Wd), _ptr(Wu), _ptr(kc), _ptr(ub),
                              _ptr(bb), _ptr(uf), _ptr(bf), _ptr(w), _ptr(beta), _ptr(logf),
                              _ptr(workspace), workspace.numel(), _stream(dev)))
    return w, beta, logf

