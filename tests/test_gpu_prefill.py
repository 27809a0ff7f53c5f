"""GPU parity of the prefill forward against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import check

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pa():
    import dependent_position_encoding_amd as pa
    pa.load_library()
    return pa


def _run(wl, L=None, block=0, variant=0, heads=None, rows=None, x=None):
    pa = _pa()
    x = workloads.make_inputs(wl, device="cpu", variant=variant, L=L) if x is None else x
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    print(f"case {wl.name} L={x['q'].shape[2]} block={block} heads={heads} rows={None if rows is None else len(rows)}", flush=True)
    o, lse = pa.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"],
                    scale=wl.scale, block=block)
    torch.cuda.synchronize()
    f64 = {k: (workloads.as_slices_f64(v, heads) if v is not None else None) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=rows)
    go = workloads.as_slices_f64(o, heads)
    gl = workloads.as_slices_f64(lse, heads)
    if rows is not None:
        rr = np.asarray(rows)
        if rr.ndim == 1:
            go, gl = go[:, rr], gl[:, rr]
        else:
            idx = np.arange(rr.shape[0])[:, None]
            go, gl = go[idx, rr], gl[idx, rr]
    return go, gl, ro, rl


@pytest.mark.parametrize("block", [16, 32, 64])
def test_tiny_fp32(block):
    wl = workloads.CONFIGS["tiny"]
    go, gl, ro, rl = _run(wl, block=block)
    check(f"tiny B={block} o", go, ro, bf16=False)
    check(f"tiny B={block} lse", gl, rl, bf16=False)


@pytest.mark.parametrize("L", [1, 2, 61, 65, 200])
def test_ragged_fp32(L):
    wl = workloads.CONFIGS["tiny"].replace(H=3)
    for block in (16, 64):
        go, gl, ro, rl = _run(wl, L=L, block=block)
        check(f"ragged L={L} B={block} o", go, ro, bf16=False)
        check(f"ragged L={L} B={block} lse", gl, rl, bf16=False)


def test_fp32_fox_and_reflections():
    wl = workloads.CONFIGS["tiny"].replace(H=2, L=300, d=32, fox=True, scale=32 ** -0.5)
    go, gl, ro, rl = _run(wl)
    check("fp32 fox o", go, ro, bf16=False)
    check("fp32 fox lse", gl, rl, bf16=False)
    st = workloads.stress(wl)
    go, gl, ro, rl = _run(st)
    check("fp32 stress o", go, ro, bf16=False)
    check("fp32 stress lse", gl, rl, bf16=False)


def test_block_size_invariance_fp32():
    pa = _pa()
    wl = workloads.CONFIGS["tiny"].replace(H=2, L=256, d=64, fox=True)
    x = workloads.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    outs = [pa.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"], scale=0.125,
                   block=b) for b in (16, 32, 64)]
    for o, lse in outs[1:]:
        assert (o - outs[0][0]).abs().max().item() < 2e-5
        assert (lse - outs[0][1]).abs().max().item() < 2e-5


def test_flipflop_bf16_full():
    wl = workloads.CONFIGS["flipflop"]
    go, gl, ro, rl = _run(wl)
    check("flipflop o", go, ro, bf16=True)
    check("flipflop lse", gl, rl, bf16=True)


def _sample_rows(L, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 63, 64, L - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, L, n - len(fixed))]))


def test_lm_bf16_sampled():
    wl = workloads.CONFIGS["lm"]
    NH = wl.N * wl.H
    heads = list(range(0, NH, 8))
    rows = _sample_rows(wl.L, 48, 3)
    go, gl, ro, rl = _run(wl, heads=heads, rows=rows)
    check("lm o", go, ro, bf16=True)
    check("lm lse", gl, rl, bf16=True)


def test_lm_bf16_scale_rsqrt_d():
    wl = workloads.CONFIGS["lm"].replace(N=1, H=8, L=1024, scale=0.125)
    go, gl, ro, rl = _run(wl, heads=[0, 3, 7])
    check("lm 1/sqrt(d) o", go, ro, bf16=True)
    check("lm 1/sqrt(d) lse", gl, rl, bf16=True)


@pytest.mark.parametrize("L", [2048])
def test_fox_bf16_sampled(L):
    wl = workloads.CONFIGS["fox"].replace(L=L)
    heads = list(range(5, wl.N * wl.H, 64))
    rows = _sample_rows(L, 48, 4)
    go, gl, ro, rl = _run(wl, heads=heads, rows=rows)
    check(f"fox L={L} o", go, ro, bf16=True)
    check(f"fox L={L} lse", gl, rl, bf16=True)


def test_bf16_ragged_and_stress():
    wl = workloads.stress(workloads.CONFIGS["fox"].replace(N=2, H=2, L=777))
    go, gl, ro, rl = _run(wl)
    check("bf16 ragged stress o", go, ro, bf16=True)
    check("bf16 ragged stress lse", gl, rl, bf16=True)


@pytest.mark.parametrize("L", [4096, 8192])
def test_fox_bf16_full_size_sampled(L):
    """The benchmark's FoX shapes (32 x 32 heads) with inputs drawn on the GPU."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(L=L)
    x = workloads.make_inputs(wl, device=DEV)
    print(f"case fox full L={L}", flush=True)
    o, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=x["logf"], scale=wl.scale)
    torch.cuda.synchronize()
    heads = list(range(7, wl.N * wl.H, 128))
    rows = _sample_rows(L, 32, L)
    f64 = {k: workloads.as_slices_f64(v, heads) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=rows)
    check(f"fox full L={L} o", workloads.as_slices_f64(o, heads)[:, rows], ro, bf16=True)
    check(f"fox full L={L} lse", workloads.as_slices_f64(lse, heads)[:, rows], rl, bf16=True)


@pytest.mark.parametrize("name,L,d", [("flipflop", 512, 32), ("lm", 1000, 64), ("lm", 4096, 64)])
def test_causal_baseline_matches_oracle_at_beta_zero(name, L, d):
    """The beta = 0 baseline kernel against the oracle with every beta = 0."""
    pa = _pa()
    wl = workloads.CONFIGS[name].replace(N=2, H=3, L=L, d=d)
    x = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    print(f"case causal {name} L={L} d={d}", flush=True)
    o, lse = pa.causal_attn(g["q"], g["k"], g["v"], scale=wl.scale)
    torch.cuda.synchronize()
    f64 = {k: workloads.as_slices_f64(v) for k, v in x.items() if v is not None}
    rows = None if L <= 1000 else _sample_rows(L, 64, 9)
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], np.zeros_like(f64["beta"]),
                             None, wl.scale, rows=rows)
    go, gl = workloads.as_slices_f64(o), workloads.as_slices_f64(lse)
    if rows is not None:
        go, gl = go[:, rows], gl[:, rows]
    check(f"causal {name} L={L} o", go, ro, bf16=True)
    check(f"causal {name} L={L} lse", gl, rl, bf16=True)


def test_causal_baseline_rejects_fp32():
    pa = _pa()
    z = torch.zeros(1, 1, 64, 64, device=DEV)
    with pytest.raises(pa.PathAttnError) as e:
        pa.causal_attn(z, z, z)
    assert e.value.status == 4
