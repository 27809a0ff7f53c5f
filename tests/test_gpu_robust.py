"""Robustness of the library's kernels on the GPU, through the C ABI:

* workspace contents never leak into results: a workspace filled with NaN
  bytes gives results bit-identical to a zeroed one (prefill, decode, paged
  decode, backward);
* nothing is written outside the outputs and cache slots a call owns: guard
  bands of a byte pattern around o, lse, gradients and cache tensors, and
  cache slots past the ones a call writes, keep the pattern;
* repeated calls are bitwise deterministic;
* decoding can be checkpointed and resumed: a cache copied to new memory
  halfway through and decoded on continues bit for bit as the original.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PATTERN = 0xA5
BAND = 512          # bytes of guard band on each side (keeps 16-byte alignment)


def _pa():
    import dependent_position_encoding_amd as pa
    pa.load_library()
    return pa


class Banded:
    """A tensor with guard bands of PATTERN bytes before and after it."""

    def __init__(self, shape, dtype, fill=PATTERN):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((n + 2 * BAND,), fill, dtype=torch.uint8, device=DEV)
        self.t = self.raw[BAND:BAND + n].view(dtype).view(shape)
        self.n = n

    def bands_intact(self):
        return bool((self.raw[:BAND] == PATTERN).all()) and bool(
            (self.raw[BAND + self.n:] == PATTERN).all())


def _poisoned(nbytes):
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=DEV)   # NaN bytes


def _zeroed(nbytes):
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV)


def _banded_cache(pa, N, H, cap, d, dtype, k_dtype, gate):
    """A Cache whose tensors sit between guard bands and start as PATTERN bytes."""
    c = pa.Cache(N, H, 1, d, dtype=dtype, k_dtype=k_dtype, gate=gate, device=DEV)
    bands = [Banded((N, H, cap, d), k_dtype), Banded((N, H, cap, d), dtype)]
    c.kcache, c.vcache = bands[0].t, bands[1].t
    if gate:
        bands.append(Banded((N, H, cap), torch.float32))
        c.gcache = bands[2].t
    c.cap = cap
    return c, bands


@pytest.mark.parametrize("dtype,d,fox", [(torch.bfloat16, 64, True), (torch.bfloat16, 32, False),
                                         (torch.float32, 32, True)])
def test_prefill_workspace_bands_and_repeats(dtype, d, fox):
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=2, H=3, L=700, d=d, dtype=dtype, fox=fox)
    x = {k: (v.to(DEV) if v is not None else None)
         for k, v in workloads.make_inputs(wl, L=wl.L).items()}
    N, H, L = wl.N, wl.H, wl.L
    cap = L + 37
    print(f"case prefill robust {dtype} d={d} fox={fox}", flush=True)
    nbytes = pa.fwd_workspace_bytes(N, H, L, d, dtype, with_cache=True)
    ref_c, _ = _banded_cache(pa, N, H, cap, d, dtype, dtype, fox)
    ref = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=x["logf"], scale=wl.scale,
                 cache=ref_c, workspace=_zeroed(nbytes))
    torch.cuda.synchronize()
    for rep in range(3):
        o, lse = Banded((N, H, L, d), dtype), Banded((N, H, L), torch.float32)
        c, cb = _banded_cache(pa, N, H, cap, d, dtype, dtype, fox)
        pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=x["logf"], scale=wl.scale,
               cache=c, workspace=_poisoned(nbytes), out=(o.t, lse.t))
        torch.cuda.synchronize()
        assert torch.equal(o.t, ref[0]) and torch.equal(lse.t, ref[1]), f"repeat {rep} differs"
        assert torch.equal(c.kcache[:, :, :L], ref_c.kcache[:, :, :L])
        assert torch.equal(c.vcache[:, :, :L], ref_c.vcache[:, :, :L])
        if fox:
            assert torch.equal(c.gcache[:, :, :L], ref_c.gcache[:, :, :L])
        assert o.bands_intact() and lse.bands_intact(), "write outside o / lse"
        assert all(b.bands_intact() for b in cb), "write outside the cache tensors"
        # slots past the prompt are not the prefill's to write
        for b in cb:
            tail = b.t[:, :, L:].contiguous().view(torch.uint8)
            assert bool((tail == PATTERN).all()), "prefill wrote past slot L - 1"


def _prefilled_cache(pa, wl, x, L, cap, k_dtype):
    c = pa.Cache(wl.N, wl.H, cap, wl.d, dtype=wl.dtype, k_dtype=k_dtype, gate=wl.fox, device=DEV)
    pre = lambda n: x[n][:, :, :L].contiguous()
    pa.fwd(pre("q"), pre("k"), pre("v"), pre("w"), pre("beta"),
           logf=pre("logf") if wl.fox else None, scale=wl.scale, cache=c)
    return c


def _copy_cache(pa, c):
    d = pa.Cache(c.N, c.H, 1, c.d, dtype=c.dtype, k_dtype=c.k_dtype, gate=c.gcache is not None,
                 device=DEV)
    d.kcache, d.vcache = c.kcache.clone(), c.vcache.clone()
    d.gcache = c.gcache.clone() if c.gcache is not None else None
    d.cap = c.cap
    return d


def _tok(x, t, fox):
    names = ("q", "k", "v", "w", "beta") + (("logf",) if fox else ())
    out = [x[n][:, :, t].contiguous() for n in names]
    return out + ([] if fox else [None])


@pytest.mark.parametrize("k_dtype", [torch.bfloat16, torch.float32])
def test_decode_workspace_bands_and_unused_slots(k_dtype):
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=2, H=3, L=500)
    steps = 4
    x = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, L=wl.L + steps).items()}
    L, cap = wl.L, wl.L + steps + 70
    print(f"case decode robust keys {k_dtype}", flush=True)
    a = _prefilled_cache(pa, wl, x, L, cap, k_dtype)
    b, bands = _banded_cache(pa, wl.N, wl.H, cap, wl.d, wl.dtype, k_dtype, True)
    b.kcache.copy_(a.kcache)
    b.vcache.copy_(a.vcache)
    b.gcache.copy_(a.gcache)
    # slots from L on: PATTERN in b; the steps write slots L .. L + steps - 1
    for t_ in (b.kcache, b.vcache, b.gcache):
        t_[:, :, L:].view(torch.uint8).fill_(PATTERN)
    nbytes = pa.decode_workspace_bytes(a, L + steps)
    for t in range(L, L + steps):
        ro, rl = pa.decode_step(a, t, *_tok(x, t, True), scale=wl.scale,
                                workspace=_zeroed(nbytes))
        o, lse = Banded((wl.N, wl.H, wl.d), wl.dtype), Banded((wl.N, wl.H), torch.float32)
        pa.decode_step(b, t, *_tok(x, t, True), scale=wl.scale, workspace=_poisoned(nbytes),
                       out=(o.t, lse.t))
        torch.cuda.synchronize()
        assert torch.equal(o.t, ro) and torch.equal(lse.t, rl), f"step {t} differs"
        assert o.bands_intact() and lse.bands_intact()
    for ta, tb, band in zip((a.kcache, a.vcache, a.gcache), (b.kcache, b.vcache, b.gcache), bands):
        n = L + steps
        assert torch.equal(ta[:, :, :n], tb[:, :, :n])
        assert bool((tb[:, :, n:].contiguous().view(torch.uint8) == PATTERN).all()), \
            "a step wrote past its slot"
        assert band.bands_intact()


@pytest.mark.parametrize("k_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fox", [True, False])
def test_decode_split_and_resume(k_dtype, fox):
    """Checkpoint / resume: 2K steps on one cache equal K steps, a copy of
    the cache into new memory, and K more steps on the copy, bit for bit."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=1, H=4, L=400, fox=fox)
    K = 5
    x = {k: (v.to(DEV) if v is not None else None)
         for k, v in workloads.make_inputs(wl, L=wl.L + 2 * K).items()}
    L, cap = wl.L, wl.L + 2 * K
    print(f"case split/resume keys {k_dtype} fox={fox}", flush=True)
    whole = _prefilled_cache(pa, wl, x, L, cap, k_dtype)
    ref = [pa.decode_step(whole, t, *_tok(x, t, fox), scale=wl.scale)
           for t in range(L, L + 2 * K)]
    first = _prefilled_cache(pa, wl, x, L, cap, k_dtype)
    got = [pa.decode_step(first, t, *_tok(x, t, fox), scale=wl.scale) for t in range(L, L + K)]
    torch.cuda.synchronize()
    resumed = _copy_cache(pa, first)
    del first
    torch.cuda.synchronize()
    got += [pa.decode_step(resumed, t, *_tok(x, t, fox), scale=wl.scale)
            for t in range(L + K, L + 2 * K)]
    torch.cuda.synchronize()
    for i, ((o, l), (ro, rl)) in enumerate(zip(got, ref)):
        assert torch.equal(o, ro) and torch.equal(l, rl), f"step {i} differs after resume"
    assert torch.equal(resumed.kcache, whole.kcache)
    assert torch.equal(resumed.vcache, whole.vcache)
    if fox:
        assert torch.equal(resumed.gcache, whole.gcache)


def test_paged_workspace_and_bands():
    pa = _pa()
    from tests.test_gpu_paged import Batch
    wl = workloads.CONFIGS["fox"].replace(N=1, H=3)
    lens = [0, 1, 64, 257, 700]
    print("case paged robust", flush=True)
    a = Batch(wl, lens, 3, 64, torch.bfloat16, seed=5)
    b = Batch(wl, lens, 3, 64, torch.bfloat16, seed=5)
    S, H, d = len(lens), wl.H, wl.d
    nbytes = pa.paged_decode_workspace_bytes(S, H, d, wl.dtype, a.max_keys)
    for i in range(3):
        t = a.token(i)
        ro, rl = pa.paged_decode_step(a.cache, a.table, a.seq_lens, a.max_keys, t["q"], t["k"],
                                      t["v"], t["w"], t["beta"], t["logf"], scale=wl.scale,
                                      workspace=_zeroed(nbytes))
        o, lse = Banded((S, H, d), wl.dtype), Banded((S, H), torch.float32)
        pa.paged_decode_step(b.cache, b.table, b.seq_lens, b.max_keys, t["q"], t["k"], t["v"],
                             t["w"], t["beta"], t["logf"], scale=wl.scale,
                             workspace=_poisoned(nbytes), out=(o.t, lse.t))
        torch.cuda.synchronize()
        assert torch.equal(o.t, ro) and torch.equal(lse.t, rl), f"paged step {i} differs"
        assert o.bands_intact() and lse.bands_intact()
    assert torch.equal(a.cache.kpages, b.cache.kpages)
    assert torch.equal(a.cache.vpages, b.cache.vpages)
    assert torch.equal(a.cache.gpages, b.cache.gpages)
    assert torch.equal(a.seq_lens, b.seq_lens)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.bfloat16, 32),
                                     (torch.float32, 16)])
def test_bwd_workspace_bands_and_repeats(dtype, d):
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=1, H=3, L=300, d=d, dtype=dtype)
    x = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, L=wl.L).items()}
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    do = torch.randn(x["q"].shape, generator=gen, device=DEV).to(dtype)
    print(f"case bwd robust {dtype} d={d}", flush=True)
    o, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=x["logf"], scale=wl.scale)
    args = (x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], o, lse, do)
    nbytes = pa.bwd_workspace_bytes(wl.N, wl.H, wl.L, d, dtype)
    ref = pa.bwd(*args, scale=wl.scale, workspace=_zeroed(nbytes))
    torch.cuda.synchronize()
    full, row = (wl.N, wl.H, wl.L, d), (wl.N, wl.H, wl.L)
    for rep in range(2):
        outs = [Banded(full, dtype) for _ in range(4)] + [Banded(row, torch.float32)
                                                         for _ in range(2)]
        pa.bwd(*args, scale=wl.scale, workspace=_poisoned(nbytes), out=[b.t for b in outs])
        torch.cuda.synchronize()
        for name, b, r in zip(("dq", "dk", "dv", "dw", "dbeta", "dlogf"), outs, ref):
            assert torch.equal(b.t, r), f"{name} differs (repeat {rep})"
            assert b.bands_intact(), f"write outside {name}"


def test_binding_rejects_mismatched_cache_and_outputs():
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=1, H=2, L=64)
    x = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, L=64).items()}
    args = (x["q"], x["k"], x["v"], x["w"], x["beta"])
    for kw in (dict(N=2), dict(H=3), dict(d=32), dict(dtype=torch.float32)):
        shape = dict(N=1, H=2, cap=64, d=64, dtype=torch.bfloat16)
        shape.update(kw)
        c = pa.Cache(shape["N"], shape["H"], shape["cap"], shape["d"], dtype=shape["dtype"],
                     device=DEV)
        with pytest.raises(ValueError):
            pa.fwd(*args, logf=x["logf"], scale=1.0, cache=c)
    o_bad = torch.empty(1, 2, 64, 32, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(1, 2, 64, device=DEV)
    with pytest.raises(ValueError):
        pa.fwd(*args, logf=x["logf"], out=(o_bad, lse))
    with pytest.raises(ValueError):
        pa.fwd(*args, logf=x["logf"], out=(torch.empty_like(x["q"]), lse.double()))
    with pytest.raises(ValueError):
        pa.fwd(*args, logf=x["logf"], workspace=torch.empty(1 << 20, device=DEV))   # not bytes
    c = pa.Cache(1, 2, 80, 64, dtype=torch.bfloat16, device=DEV)
    tok = [x[n][:, :, 0].contiguous() for n in ("q", "k", "v", "w", "beta", "logf")]
    with pytest.raises(ValueError):
        pa.decode_step(c, 0, *tok, out=(torch.empty(1, 2, 64, device=DEV), None))
    src = pa.Cache(1, 2, 80, 64, dtype=torch.bfloat16, k_dtype=torch.float32, device=DEV)
    dst = pa.PagedCache(4, 64, 2, 64, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(1, 2, dtype=torch.int32, device=DEV)
    lens = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        pa.paged_import(src, dst, table, lens, 80)
