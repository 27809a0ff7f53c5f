"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments synchronously (no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "path_attn.h")).read()
    return sorted(set(re.findall(r"\b(path_[a-z_0-9]+)\s*\(", src)))


def _lib():
    import dependent_position_encoding_amd as pa
    return pa, pa.load_library()


def test_every_declared_symbol_is_exported():
    pa, lib = _lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pa.EXPORTS) == names


def test_abi_version_and_status_strings():
    pa, lib = _lib()
    assert lib.path_abi_version() == 5
    for s in range(9):
        assert lib.path_status_str(s)
    assert lib.path_status_str(99) == b"unknown status"


def _desc(pa, **kw):
    base = dict(N=1, H=1, L=64, d=64, dtype=pa.PATH_BF16, scale=1.0, block=0)
    base.update(kw)
    return pa._Desc(**base)


FAKE = ctypes.c_void_p(1 << 20)     # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 2), (dict(L=0), 2), (dict(L=(1 << 23) + 1), 2), (dict(d=48), 4), (dict(d=128), 4),
    (dict(dtype=7), 3), (dict(block=8), 4), (dict(block=32), 4),
])
def test_fwd_rejects_bad_descriptions(kw, status):
    pa, lib = _lib()
    d = _desc(pa, **kw)
    st = lib.path_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                           None, FAKE, 1 << 30, None)
    assert st == status
    assert lib.path_last_error()
    assert lib.path_attn_fwd_workspace(ctypes.byref(d), 0) == 0


def test_fwd_rejects_null_misaligned_and_small_workspace():
    pa, lib = _lib()
    d = _desc(pa)
    st = lib.path_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, 0, None)
    assert st == 1
    st = lib.path_attn_fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, 0, None)
    assert st == 1
    odd = ctypes.c_void_p((1 << 20) + 2)
    st = lib.path_attn_fwd(ctypes.byref(d), odd, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, 0, None)
    assert st == 5
    need = lib.path_attn_fwd_workspace(ctypes.byref(d), 0)
    assert need > 0
    assert lib.path_attn_fwd_workspace(ctypes.byref(d), 1) > need
    st = lib.path_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                           FAKE, need - 1, None)
    assert st == 6
    st = lib.path_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                           None, need, None)
    assert st == 6
    st = lib.path_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                           ctypes.c_void_p((1 << 20) + 16), need, None)
    assert st == 5


def test_fwd_cache_capacity_checked():
    pa, lib = _lib()
    d = _desc(pa, L=100)
    c = pa._Cache(99, pa.PATH_BF16, 1 << 20, 1 << 21, None)
    need = lib.path_attn_fwd_workspace(ctypes.byref(d), 1)
    st = lib.path_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                           ctypes.byref(c), FAKE, need, None)
    assert st == 7


def test_decode_argument_errors():
    pa, lib = _lib()
    d = _desc(pa)
    c = pa._Cache(8, pa.PATH_BF16, 1 << 20, 1 << 21, None)
    ws = lib.path_decode_workspace(ctypes.byref(d), 8)
    assert ws > 0
    assert lib.path_decode(ctypes.byref(d), ctypes.byref(c), 9, FAKE, FAKE, None, FAKE, ws, None) == 7
    assert lib.path_decode(ctypes.byref(d), ctypes.byref(c), 0, FAKE, FAKE, None, FAKE, ws, None) == 2
    assert lib.path_decode(ctypes.byref(d), None, 4, FAKE, FAKE, None, FAKE, ws, None) == 1
    assert lib.path_decode(ctypes.byref(d), ctypes.byref(c), 4, FAKE, FAKE, None, FAKE, 8, None) == 6
    assert lib.path_decode_step(ctypes.byref(d), ctypes.byref(c), 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None, FAKE, None, FAKE, ws, None) == 7
    assert lib.path_kv_update(ctypes.byref(d), ctypes.byref(c), 9, FAKE, FAKE, None) == 7
    assert lib.path_kv_update(ctypes.byref(d), ctypes.byref(c), -1, FAKE, FAKE, None) == 2
    assert lib.path_kv_append(ctypes.byref(d), ctypes.byref(c), 8, FAKE, FAKE, None, None) == 7
    g = pa._Cache(8, pa.PATH_BF16, 1 << 20, 1 << 21, 1 << 22)
    assert lib.path_kv_append(ctypes.byref(d), ctypes.byref(g), 0, FAKE, FAKE, None, None) == 1
    bad = pa._Cache(8, 5, 1 << 20, 1 << 21, None)
    assert lib.path_kv_update(ctypes.byref(d), ctypes.byref(bad), 1, FAKE, FAKE, None) == 3


def test_param_argument_errors():
    """The front-end rejects bad descriptions, missing or mismatched gate
    arguments, misaligned pointers and small workspaces before any launch."""
    pa, lib = _lib()
    P = lambda **kw: pa._ParamDesc(**{**dict(N=1, L=64, Dm=64, R=16, H=2, d=64,
                                               dtype=pa.PATH_BF16), **kw})
    good = P()
    ws = lib.path_param_workspace(ctypes.byref(good), 1)
    assert ws >= 64 * 32 * 4 and ws % 256 == 0
    assert lib.path_param_workspace(ctypes.byref(P(R=8)), 1) == 0
    args = lambda d, **kw: [ctypes.byref(d)] + [kw.get(n, FAKE) for n in (
        "x", "Wd", "Wu", "kc", "ub", "bb", "uf", "bf", "w", "beta", "logf", "ws")] + [
        kw.get("ws_bytes", ws), None]
    for kw, status in [(dict(N=0), 2), (dict(d=48), 4), (dict(Dm=40), 4), (dict(R=8), 4),
                       (dict(R=272), 4), (dict(dtype=7), 3), (dict(Dm=65552), 4),
                       (dict(L=1 << 24), 2)]:
        assert lib.path_param_fwd(*args(P(**kw))) == status, kw
    assert lib.path_param_fwd(*args(good, x=None)) == 1
    assert lib.path_param_fwd(*args(good, uf=None)) == 1                # gate args must match
    assert lib.path_param_fwd(*args(good, uf=None, bf=None, logf=None, ws_bytes=8)) == 6
    assert lib.path_param_fwd(*args(good, x=ctypes.c_void_p((1 << 20) + 8))) == 5
    assert lib.path_param_fwd(*args(good, ws=ctypes.c_void_p((1 << 20) + 64))) == 5
    assert lib.path_param_fwd(*args(good, ws_bytes=ws - 256)) == 6



def _paged(pa, **kw):
    base = dict(num_pages=8, page_size=64, k_dtype=pa.PATH_BF16, kpages=FAKE.value,
                vpages=FAKE.value, gpages=None)
    base.update(kw)
    return pa._PagedCache(**base)


def _paged_step(pa, lib, d, pc, stride=4, max_keys=256, ws_bytes=1 << 30, ws=FAKE, q=FAKE,
                logf=None):
    return lib.path_paged_decode_step(ctypes.byref(d), ctypes.byref(pc) if pc else None, FAKE,
                                      stride, FAKE, max_keys, q, FAKE, FAKE, FAKE, FAKE, logf,
                                      FAKE, None, ws, ws_bytes, None)


def test_paged_argument_errors():
    pa, lib = _lib()
    d = _desc(pa, N=3, H=2)
    assert _paged_step(pa, lib, d, None) == 1
    assert _paged_step(pa, lib, d, _paged(pa), q=None) == 1
    assert _paged_step(pa, lib, d, _paged(pa, gpages=FAKE.value)) == 1     # logf_t missing
    for ps in (8, 48, 256):
        assert _paged_step(pa, lib, d, _paged(pa, page_size=ps)) == 4
    assert _paged_step(pa, lib, d, _paged(pa, num_pages=0)) == 2
    assert _paged_step(pa, lib, d, _paged(pa, k_dtype=5)) == 3
    assert _paged_step(pa, lib, d, _paged(pa), max_keys=0) == 2
    assert _paged_step(pa, lib, d, _paged(pa), max_keys=131073, stride=4096) == 4
    assert _paged_step(pa, lib, d, _paged(pa), max_keys=257, stride=4) == 2   # 5 pages needed
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert _paged_step(pa, lib, d, _paged(pa, kpages=odd.value)) == 5
    need = lib.path_paged_decode_workspace(ctypes.byref(d), 256)
    assert need > 0 and lib.path_paged_decode_workspace(ctypes.byref(d), 0) == 0
    assert _paged_step(pa, lib, d, _paged(pa), ws_bytes=need - 1) == 6
    assert _paged_step(pa, lib, d, _paged(pa), ws=None, ws_bytes=need) == 6
    assert _paged_step(pa, lib, _desc(pa, N=3, H=2, d=48), _paged(pa)) == 4
    # import: dtype and gate consistency are checked before any launch
    src = pa._Cache(512, pa.PATH_F32, FAKE.value, FAKE.value, None)
    st = lib.path_paged_import(ctypes.byref(d), ctypes.byref(src), ctypes.byref(_paged(pa)),
                               FAKE, 4, FAKE, 256, None)
    assert st == 3
    src = pa._Cache(512, pa.PATH_BF16, FAKE.value, FAKE.value, FAKE.value)
    st = lib.path_paged_import(ctypes.byref(d), ctypes.byref(src), ctypes.byref(_paged(pa)),
                               FAKE, 4, FAKE, 256, None)
    assert st == 1
    st = lib.path_paged_import(ctypes.byref(d), ctypes.byref(src), ctypes.byref(_paged(pa)),
                               None, 4, FAKE, 256, None)
    assert st == 1


def _bwd_args(pa, lib, d, **kw):
    """Arguments of path_attn_bwd: every tensor a fake aligned pointer unless overridden."""
    names = ("q", "k", "v", "w", "beta", "logf", "o", "lse", "dout", "dq", "dk", "dv", "dw",
             "dbeta", "dlogf", "ws")
    ws_bytes = kw.pop("ws_bytes", 1 << 40)
    return [ctypes.byref(d) if d is not None else None] + [kw.get(n, FAKE) for n in names] + [
        ws_bytes, None]


def test_bwd_argument_errors():
    pa, lib = _lib()
    d = _desc(pa, N=2, H=3, L=200)
    need = lib.path_attn_bwd_workspace(ctypes.byref(d))
    assert need > 0 and need % 256 == 0
    # block must be 64 for the backward; invalid descriptions size to 0
    for kw in (dict(block=32, dtype=pa.PATH_F32), dict(N=0), dict(d=48), dict(dtype=9)):
        assert lib.path_attn_bwd_workspace(ctypes.byref(_desc(pa, **kw))) == 0, kw
    assert lib.path_attn_bwd_workspace(None) == 0
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, None)) == 1
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, _desc(pa, block=32, dtype=pa.PATH_F32))) == 4
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, _desc(pa, d=128))) == 4
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, _desc(pa, L=0))) == 2
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, _desc(pa, dtype=9))) == 3
    for n in ("q", "k", "v", "w", "beta", "o", "lse", "dout", "dq", "dk", "dv", "dw", "dbeta"):
        assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, **{n: None})) == 1, n
    # the gate input and its gradient come together
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, logf=None)) == 1
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, dlogf=None)) == 1
    odd16 = ctypes.c_void_p((1 << 20) + 8)
    odd4 = ctypes.c_void_p((1 << 20) + 2)
    for n in ("q", "k", "v", "w", "o", "dout", "dq", "dk", "dv", "dw"):
        assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, **{n: odd16})) == 5, n
    for n in ("beta", "logf", "lse", "dbeta", "dlogf"):
        assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, **{n: odd4})) == 5, n
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, ws=None, ws_bytes=need)) == 6
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, ws_bytes=need - 1)) == 6
    assert lib.path_attn_bwd(*_bwd_args(pa, lib, d, ws=ctypes.c_void_p((1 << 20) + 128),
                                        ws_bytes=need)) == 5
    assert lib.path_last_error()


def test_causal_argument_errors():
    pa, lib = _lib()
    call = lambda d, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None: lib.path_causal_attn_fwd(
        ctypes.byref(d) if d is not None else None, q, k, v, o, lse, None)
    assert call(None) == 1
    assert call(_desc(pa), q=None) == 1
    assert call(_desc(pa), o=None) == 1
    assert call(_desc(pa, N=0)) == 2
    assert call(_desc(pa, dtype=9)) == 3
    assert call(_desc(pa, dtype=pa.PATH_F32)) == 4      # baseline is bf16 only
    assert call(_desc(pa, d=16)) == 4                   # head dim 32 or 64
    assert call(_desc(pa), v=ctypes.c_void_p((1 << 20) + 8)) == 5
    assert lib.path_last_error()


def test_fwd_timed_argument_errors():
    pa, lib = _lib()
    d = _desc(pa)
    need = lib.path_attn_fwd_workspace(ctypes.byref(d), 0)
    args = [ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, need, None]
    assert lib.path_attn_fwd_timed(*args, None) == 1
    evs = (ctypes.c_void_p * 4)(1, 2, 0, 4)           # one event missing
    assert lib.path_attn_fwd_timed(*args, evs) == 1
    evs = (ctypes.c_void_p * 4)(1, 2, 3, 4)           # never recorded: validation fails first
    bad = list(args)
    bad[0] = ctypes.byref(_desc(pa, d=48))
    assert lib.path_attn_fwd_timed(*bad, evs) == 4
    bad = list(args)
    bad[11] = need - 1
    assert lib.path_attn_fwd_timed(*bad, evs) == 6
    assert lib.path_last_error()


def test_noalloc_step_argument_errors():
    """The allocation-free decode step validates exactly as path_decode_step
    does, and refuses a step whose partial states exceed its static scratch,
    all before anything touches a device."""
    pa, lib = _lib()
    limit = lib.path_decode_step_noalloc_limit()
    assert limit == 16 << 20
    d = _desc(pa)
    c = pa._Cache(8, pa.PATH_BF16, 1 << 20, 1 << 21, None)
    call = lambda desc, cache, n, **kw: lib.path_decode_step_noalloc(
        ctypes.byref(desc) if desc is not None else None, ctypes.byref(cache) if cache else None,
        n, *[kw.get(x, FAKE) for x in ("q", "k", "v", "w", "beta")], kw.get("logf"),
        kw.get("o", FAKE), None, None)
    assert call(None, c, 2) == 1
    assert call(d, None, 2) == 1
    assert call(d, c, 8) == 7                  # slot 8 of a cache of 8
    assert call(d, c, -1) == 2
    assert call(d, c, 2, q=None) == 1
    assert call(d, c, 2, k=ctypes.c_void_p((1 << 20) + 8)) == 5
    assert call(_desc(pa, d=48), c, 2) == 4
    g = pa._Cache(8, pa.PATH_BF16, 1 << 20, 1 << 21, 1 << 22)
    assert call(d, g, 2) == 1                  # gate prefix without log f_t
    # 4096 slices x 1024 chunks of partial states: far beyond the scratch
    big = _desc(pa, N=64, H=64)
    cb = pa._Cache(131072, pa.PATH_BF16, 1 << 20, 1 << 21, None)
    assert lib.path_decode_workspace(ctypes.byref(big), 131072) > limit
    assert call(big, cb, 131071) == 6
    assert b"static scratch" in lib.path_last_error()
