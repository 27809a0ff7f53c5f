"""GPU parity of the decode path: cache alignment after prefill, the cache
rewrite, and single-query attention, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import check, check_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pa():
    import dependent_position_encoding_amd as pa
    pa.load_library()
    return pa


def _decode_run(wl, L, steps, k_dtype, fused=True, variant=0):
    """Prefill L tokens into a cache, then decode `steps` tokens.

    Returns the GPU outputs and the fp64 oracle rows for positions
    L .. L+steps-1 (rows of the walk on the whole sequence), and the final
    cache keys with their oracle.
    """
    pa = _pa()
    x = workloads.make_inputs(wl, device="cpu", variant=variant, L=L + steps)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    N, H, d = wl.N, wl.H, wl.d
    gate = wl.fox
    print(f"case {wl.name} L={L} steps={steps} k_dtype={k_dtype} fused={fused}", flush=True)
    cache = pa.Cache(N, H, L + steps, d, dtype=wl.dtype, k_dtype=k_dtype, gate=gate, device=DEV)
    pre = lambda n: g[n][:, :, :L].contiguous()
    pa.fwd(pre("q"), pre("k"), pre("v"), pre("w"), pre("beta"),
           logf=pre("logf") if gate else None, scale=wl.scale, cache=cache)
    outs, lses = [], []
    tok = lambda n, t: g[n][:, :, t].contiguous()
    for t in range(L, L + steps):
        lf = tok("logf", t) if gate else None
        if fused:
            o, lse = pa.decode_step(cache, t, tok("q", t), tok("k", t), tok("v", t), tok("w", t),
                                    tok("beta", t), lf, scale=wl.scale)
        else:
            pa.kv_update(cache, t, tok("w", t), tok("beta", t))
            pa.kv_append(cache, t, tok("k", t), tok("v", t), lf)
            o, lse = pa.decode(cache, t + 1, tok("q", t), scale=wl.scale)
        outs.append(o.clone())
        lses.append(lse.clone())
    torch.cuda.synchronize()
    go = np.stack([workloads.as_slices_f64(o) for o in outs], axis=1)
    gl = np.stack([workloads.as_slices_f64(l) for l in lses], axis=1)
    f64 = {k: (workloads.as_slices_f64(v) if v is not None else None) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"],
                             f64["logf"] if gate else None, wl.scale,
                             rows=np.arange(L, L + steps))
    kc = workloads.as_slices_f64(cache.kcache)
    rk = oracle.transported_keys(f64["k"], f64["w"], f64["beta"], L + steps - 1)
    return go, gl, ro, rl, kc, rk, cache, x


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("dtype,k_dtype", [(torch.float32, torch.float32),
                                           (torch.bfloat16, torch.bfloat16),
                                           (torch.bfloat16, torch.float32)])
def test_decode_small(dtype, k_dtype, fused):
    wl = workloads.CONFIGS["fox"].replace(N=2, H=3, L=190, dtype=dtype)
    go, gl, ro, rl, kc, rk, _, _ = _decode_run(wl, 190, 12, k_dtype, fused)
    bf = dtype == torch.bfloat16
    check("decode o", go, ro, bf16=bf)
    check("decode lse", gl, rl, bf16=bf)
    check_cache("decode kcache", kc, rk, k_dtype, 12)


@pytest.mark.parametrize("gate", [True, False])
def test_decode_bf16_head_dim_32(gate):
    """Head dim 32 on the matrix-core prefill (its own image layout and
    alignment tiles), a ragged prompt, then fused decode steps."""
    wl = workloads.CONFIGS["flipflop"].replace(N=2, H=2, L=203, fox=gate)
    go, gl, ro, rl, kc, rk, _, _ = _decode_run(wl, 203, 10, torch.bfloat16, True)
    check("d32 decode o", go, ro, bf16=True)
    check("d32 decode lse", gl, rl, bf16=True)
    check_cache("d32 decode kcache", kc, rk, torch.bfloat16, 10)


def test_decode_no_gate_and_ragged_prompt():
    wl = workloads.CONFIGS["tiny"].replace(N=1, H=2, L=77, d=32, scale=32 ** -0.5)
    go, gl, ro, rl, kc, rk, _, _ = _decode_run(wl, 77, 9, torch.float32, True)
    check("decode nogate o", go, ro, bf16=False)
    check("decode nogate lse", gl, rl, bf16=False)
    np.testing.assert_allclose(kc, rk, atol=5e-5)


def test_decode_from_empty_cache():
    """Position 0 decoded alone: o_0 = v_0 and lse_0 = scale * q_0 . k_0."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=1, H=4, L=4, dtype=torch.float32)
    x = workloads.make_inputs(wl, L=4)
    g = {k: v.to(DEV) for k, v in x.items()}
    cache = pa.Cache(1, 4, 4, 64, dtype=torch.float32, gate=True, device=DEV)
    tok = lambda n, t: g[n][:, :, t].contiguous()
    o, lse = pa.decode_step(cache, 0, tok("q", 0), tok("k", 0), tok("v", 0), tok("w", 0),
                            tok("beta", 0), tok("logf", 0), scale=0.125)
    torch.cuda.synchronize()
    assert torch.allclose(o, g["v"][:, :, 0], atol=1e-6)
    ref = 0.125 * (g["q"][:, :, 0] * g["k"][:, :, 0]).sum(-1)
    assert torch.allclose(lse, ref, atol=1e-5)
    assert torch.allclose(cache.gcache[:, :, 0], g["logf"][:, :, 0])


def test_fused_and_unfused_agree():
    wl = workloads.CONFIGS["fox"].replace(N=1, H=2, L=300)
    a = _decode_run(wl, 300, 6, torch.bfloat16, True)
    b = _decode_run(wl, 300, 6, torch.bfloat16, False)
    assert np.abs(a[0] - b[0]).max() < 1e-2
    assert np.array_equal(a[4], b[4]), "the two paths must rewrite the cache identically"


def test_cache_capacity_errors():
    pa = _pa()
    cache = pa.Cache(1, 1, 4, 16, dtype=torch.float32, gate=False, device=DEV)
    z = torch.zeros(1, 1, 16, device=DEV)
    b = torch.zeros(1, 1, device=DEV)
    with pytest.raises(pa.PathAttnError) as e:
        pa.decode_step(cache, 4, z, z, z, z, b, None)
    assert e.value.status == 7
    with pytest.raises(pa.PathAttnError) as e:
        pa.decode(cache, 5, z)
    assert e.value.status == 7


def _long_case(wl, k_dtype, head_stride=1, steps=None, check_heads=None):
    """Full-size long-context case in the launch configuration the benchmark
    times: prefill with cache alignment, then fused decode steps.  Inputs are
    drawn on the GPU (seeded); the oracle gets the sampled heads' values."""
    pa = _pa()
    steps = wl.decode_steps if steps is None else steps
    L = wl.L
    x = workloads.make_inputs(wl, device=DEV, L=L + steps)
    N, H, d = wl.N, wl.H, wl.d
    print(f"case {wl.name} full L={L} steps={steps} k_dtype={k_dtype}", flush=True)
    cache = pa.Cache(N, H, L + steps, d, dtype=wl.dtype, k_dtype=k_dtype, gate=True, device=DEV)
    pre = lambda n: x[n][:, :, :L].contiguous()
    o, lse = pa.fwd(pre("q"), pre("k"), pre("v"), pre("w"), pre("beta"), logf=pre("logf"),
                    scale=wl.scale, cache=cache)
    tok = lambda n, t: x[n][:, :, t].contiguous()
    outs, lses = [], []
    for t in range(L, L + steps):
        ot, lt = pa.decode_step(cache, t, tok("q", t), tok("k", t), tok("v", t), tok("w", t),
                                tok("beta", t), tok("logf", t), scale=wl.scale)
        outs.append(ot.clone())
        lses.append(lt.clone())
    torch.cuda.synchronize()
    heads = list(range(0, N * H, head_stride)) if check_heads is None else check_heads
    f64 = {k: workloads.as_slices_f64(v, heads) for k, v in x.items()}
    go = np.stack([workloads.as_slices_f64(o_, heads) for o_ in outs], axis=1)
    gl = np.stack([workloads.as_slices_f64(l_, heads) for l_ in lses], axis=1)
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=np.arange(L, L + steps))
    check(f"{wl.name} decode o", go, ro, bf16=True)
    check(f"{wl.name} decode lse", gl, rl, bf16=True)
    # prefill rows of 4 heads, including the first and last rows of blocks
    rows = np.unique(np.concatenate([[0, 63, 64, 4095, L - 64, L - 1],
                                     np.random.default_rng(5).integers(0, L, 40)]))
    ph = heads[:4]
    f4 = {k: workloads.as_slices_f64(v, ph) for k, v in x.items()}
    po, pl = oracle.fwd_rows(f4["q"], f4["k"], f4["v"], f4["w"], f4["beta"], f4["logf"],
                             wl.scale, rows=rows)
    check(f"{wl.name} prefill o", workloads.as_slices_f64(o, ph)[:, rows], po, bf16=True)
    check(f"{wl.name} prefill lse", workloads.as_slices_f64(lse, ph)[:, rows], pl, bf16=True)
    # the final cache: sampled slots of 2 heads against explicitly transported keys
    kh = heads[:2]
    fk = {k: workloads.as_slices_f64(v, kh) for k, v in x.items()}
    rk = oracle.transported_keys(fk["k"], fk["w"], fk["beta"], L + steps - 1)
    slots = np.unique(np.concatenate([[0, 1, L - 1, L, L + steps - 1],
                                      np.random.default_rng(6).integers(0, L + steps, 250)]))
    check_cache(f"{wl.name} kcache", workloads.as_slices_f64(cache.kcache, kh)[:, slots],
                rk[:, slots], k_dtype, steps)


def test_long_context_full_size():
    _long_case(workloads.CONFIGS["long"], torch.bfloat16)


@pytest.mark.parametrize("k_dtype", [torch.bfloat16, torch.float32])
def test_long_context_stress_full_size(k_dtype):
    """The near-reflection stress variant: all 32 heads x 256 decode steps."""
    _long_case(workloads.stress(workloads.CONFIGS["long"]), k_dtype)


def test_decode_steps_replayed_from_a_graph():
    """The fused decode steps captured in a HIP graph and replayed (with eager
    prefills in between) give exactly the eager results on every replay."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=1, H=4, L=300)
    steps = 6
    x = workloads.make_inputs(wl, device="cpu", L=wl.L + steps)
    g = {k: v.to(DEV) for k, v in x.items()}
    L = wl.L
    pre = {n: g[n][:, :, :L].contiguous() for n in g}
    tok = {n: [g[n][:, :, t].contiguous() for t in range(L, L + steps)] for n in g}
    cache = pa.Cache(1, 4, L + steps, wl.d, dtype=wl.dtype, gate=True, device=DEV)
    outs = [(torch.empty(1, 4, wl.d, dtype=wl.dtype, device=DEV),
             torch.empty(1, 4, dtype=torch.float32, device=DEV)) for _ in range(steps)]
    dws = torch.empty(pa.decode_workspace_bytes(cache, L + steps), dtype=torch.uint8, device=DEV)
    fws = torch.empty(pa.fwd_workspace_bytes(1, 4, L, wl.d, wl.dtype, with_cache=True),
                      dtype=torch.uint8, device=DEV)

    def prefill():
        pa.fwd(pre["q"], pre["k"], pre["v"], pre["w"], pre["beta"], logf=pre["logf"],
               scale=wl.scale, cache=cache, workspace=fws)

    def loop():
        for i in range(steps):
            pa.decode_step(cache, L + i, *(tok[n][i] for n in ("q", "k", "v", "w", "beta", "logf")),
                           scale=wl.scale, workspace=dws, out=outs[i])

    print("case graph replay", flush=True)
    prefill()
    loop()
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in outs]
    ref_k = cache.kcache.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        prefill()
        for o, l in outs:
            o.zero_()
            l.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(l, rl), f"replay {rep} differs"
        assert torch.equal(cache.kcache, ref_k)
