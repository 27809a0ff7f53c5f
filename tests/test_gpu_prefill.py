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


def _rows_per_head(L, heads, n, seed):
    """[len(heads), n] query rows: 0, 63, 64 and L - 1 in every head, the rest
    drawn per head (so the sampled rows of different heads hit different
    query blocks)."""
    rng = np.random.default_rng(seed)
    fixed = np.array([0, 63, 64, L - 1])
    out = np.empty((len(heads), n), dtype=np.int64)
    for i in range(len(heads)):
        rest = rng.choice(np.setdiff1d(np.arange(L), fixed), n - len(fixed), replace=False)
        out[i] = np.sort(np.concatenate([fixed, rest]))
    return out


def _check_full_size(name, x, o, lse, scale, full_heads, sampled_heads, rows):
    """Full heads (every row) and sampled rows of other heads against the oracle."""
    f64 = {k: (workloads.as_slices_f64(v, full_heads) if v is not None else None)
           for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             scale)
    check(f"{name} full heads {full_heads} o", workloads.as_slices_f64(o, full_heads), ro, bf16=True)
    check(f"{name} full heads lse", workloads.as_slices_f64(lse, full_heads), rl, bf16=True)
    f64 = {k: (workloads.as_slices_f64(v, sampled_heads) if v is not None else None)
           for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             scale, rows=rows)
    idx = np.arange(len(sampled_heads))[:, None]
    go = workloads.as_slices_f64(o, sampled_heads)[idx, rows]
    gl = workloads.as_slices_f64(lse, sampled_heads)[idx, rows]
    check(f"{name} {len(sampled_heads)} heads x {rows.shape[1]} rows o", go, ro, bf16=True)
    check(f"{name} {len(sampled_heads)} heads x {rows.shape[1]} rows lse", gl, rl, bf16=True)


def test_lm_bf16_full_size():
    """The LM-layer workload at full size (4 x 24 heads, L = 4096, d = 64):
    4 heads checked on every row, and 64 rows (0, 63, 64, L - 1 and 60 drawn
    per head) of all 96 heads."""
    pa = _pa()
    wl = workloads.CONFIGS["lm"]
    x = workloads.make_inputs(wl, device=DEV)
    print(f"case lm full {tuple(x['q'].shape)}", flush=True)
    o, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=None, scale=wl.scale)
    torch.cuda.synchronize()
    NH = wl.N * wl.H
    heads = list(range(NH))
    _check_full_size("lm", x, o, lse, wl.scale, [0, 37, 58, NH - 1], heads,
                     _rows_per_head(wl.L, heads, 64, 3))


def test_lm_bf16_scale_rsqrt_d():
    wl = workloads.CONFIGS["lm"].replace(N=1, H=8, L=1024, scale=0.125)
    go, gl, ro, rl = _run(wl, heads=[0, 3, 7])
    check("lm 1/sqrt(d) o", go, ro, bf16=True)
    check("lm 1/sqrt(d) lse", gl, rl, bf16=True)


def test_bf16_ragged_and_stress():
    wl = workloads.stress(workloads.CONFIGS["fox"].replace(N=2, H=2, L=777))
    go, gl, ro, rl = _run(wl)
    check("bf16 ragged stress o", go, ro, bf16=True)
    check("bf16 ragged stress lse", gl, rl, bf16=True)


@pytest.mark.parametrize("L", [2048, 4096, 8192])
def test_fox_bf16_full_size(L):
    """PaTH-FoX at the kernel-timing figure's shape (32 x 32 heads, d = 64)
    at L = 2048, 4096 and 8192, inputs drawn on the GPU: 16 heads x 64 rows
    (0, 63, 64, L - 1 and 60 drawn per head) and one head on every row."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(L=L)
    x = workloads.make_inputs(wl, device=DEV)
    print(f"case fox full L={L}", flush=True)
    o, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=x["logf"], scale=wl.scale)
    torch.cuda.synchronize()
    NH = wl.N * wl.H
    heads = sorted(np.random.default_rng(L).choice(NH, 16, replace=False).tolist())
    full = [int(np.random.default_rng(L + 1).integers(NH))]
    _check_full_size(f"fox L={L}", x, o, lse, wl.scale, full, heads,
                     _rows_per_head(L, heads, 64, L + 2))


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
