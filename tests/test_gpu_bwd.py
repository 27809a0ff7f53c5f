"""GPU parity of the backward pass (path_attn_bwd, through the C ABI) against
the fp64 oracle's gradients (oracle.bwd), on the same inputs: the forward's
inputs, dL/do, and the forward's own o and lse.

Bars, relative to each gradient's largest reference magnitude g_max (the
gradients are sums of many terms whose scale depends on the tensor; g_max is
taken as at least 1, so gradients smaller than that get an absolute bar):
  float32 inputs: max |err| <= 1e-4 g_max;
  bf16 inputs:    max |err| <= 2e-2 g_max and sum |err| / sum |ref| <= 1e-2.
The bf16 bar follows from the arithmetic: the rows' Delta_i = do_i . o_i
uses the forward's bf16-rounded o (relative error 2^-9 per element), which
enters every dS_ij; P and dS enter their products rounded to bf16 (2^-9),
the other fp32 operands as hi + lo parts (~16 mantissa bits); and every
gradient is itself rounded to bf16 (2^-9).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dw", "dbeta", "dlogf")


def _pa():
    import dependent_position_encoding_amd as pa
    pa.load_library()
    return pa


def _errs(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite gradient"
    gmax = max(float(np.abs(ref).max()), 1.0)   # an absolute bar for small gradients
    err = np.abs(got - ref)
    return float(err.max()) / gmax, float(err.sum() / max(np.abs(ref).sum(), 1e-300)), gmax


def _run(wl, L, seed=0):
    pa = _pa()
    x = workloads.make_inputs(wl, device="cpu", variant=seed, L=L)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1234 + seed)
    do = torch.randn(g["q"].shape, generator=gen).to(wl.dtype).to(DEV)
    print(f"case bwd {wl.name} N={wl.N} H={wl.H} L={L} d={wl.d} {wl.dtype} fox={wl.fox}",
          flush=True)
    o, lse = pa.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"], scale=wl.scale)
    grads = pa.bwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["logf"], o, lse, do,
                   scale=wl.scale)
    torch.cuda.synchronize()
    f64 = {k: (workloads.as_slices_f64(v) if v is not None else None) for k, v in x.items()}
    ref = oracle.bwd(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                     wl.scale, workloads.as_slices_f64(do))
    bf16 = wl.dtype == torch.bfloat16
    out = {}
    for name, got in zip(NAMES, grads):
        if ref[name] is None:
            assert got is None
            continue
        gm = workloads.as_slices_f64(got)
        ma, mr, gmax = _errs(gm, ref[name])
        ok = ma <= 2e-2 and mr <= 1e-2 if bf16 else ma <= 1e-4
        msg = f"  {name}: max-err/g_max {ma:.2e} mean-rel {mr:.2e} (g_max {gmax:.3g})"
        print(msg, flush=True)
        out[name] = (ok, msg)
    bad = [m for ok, m in out.values() if not ok]
    assert not bad, bad
    return grads, ref


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("fox", [False, True])
def test_bwd_fp32(d, fox):
    # three blocks, the last one ragged
    wl = workloads.CONFIGS["tiny"].replace(H=2, d=d, fox=fox, scale=d ** -0.5)
    _run(wl, L=150)


def test_bwd_fp32_one_block_and_single_token():
    wl = workloads.CONFIGS["tiny"].replace(H=2, fox=True)
    _run(wl, L=64)
    grads, ref = _run(wl, L=1)
    # one key per row: P = 1 and dS = 0 (up to the rounding of do . o against
    # do . v), so only v gets gradient, and dv = do
    for t in (grads[0], grads[1], grads[3], grads[4]):
        assert t.abs().max().item() < 1e-5


def test_bwd_fp32_near_reflections():
    wl = workloads.stress(workloads.CONFIGS["tiny"].replace(H=2, d=32, fox=True,
                                                            scale=32 ** -0.5))
    _run(wl, L=200, seed=1)


@pytest.mark.parametrize("fox", [False, True])
def test_bwd_bf16(fox):
    wl = workloads.CONFIGS["lm"].replace(N=1, H=2, fox=fox)
    _run(wl, L=150)


@pytest.mark.parametrize("fox", [False, True])
def test_bwd_bf16_head_dim_32(fox):
    """Head dim 32 (the flip-flop layer's) on the matrix-core backward kernels:
    five blocks, the last one ragged, with and without the gate."""
    wl = workloads.CONFIGS["flipflop"].replace(N=2, H=2, fox=fox)
    _run(wl, L=300, seed=4)


def test_bwd_bf16_flipflop_full_shape():
    """The flip-flop layer's full shape (16 x 2 heads, L = 512, d = 32)."""
    _run(workloads.CONFIGS["flipflop"], L=512, seed=5)


@pytest.mark.parametrize("fox", [False, True])
def test_bwd_bf16_head_dim_16(fox):
    """Head dim 16 (generic kernels, bf16 data): four blocks, ragged."""
    wl = workloads.CONFIGS["fox"].replace(N=1, H=2, d=16, qk_std=16 ** -0.25, fox=fox)
    _run(wl, L=200, seed=6)


def test_bwd_bf16_ragged_slice_group():
    # 20 slices: the pair kernels take slices 16 at a time, so one full group
    # and one of 4; a ragged sequence tail as well
    wl = workloads.CONFIGS["fox"].replace(N=2, H=10)
    _run(wl, L=300, seed=3)


def test_bwd_bf16_many_blocks():
    # 16 blocks: long transition chains through the scan's backward
    wl = workloads.CONFIGS["fox"].replace(N=1, H=2)
    _run(wl, L=1024, seed=2)


def test_bwd_bf16_full_lm_shape_sampled_slices():
    """The LM-layer training shape the benchmark times (4 x 24 heads, L =
    4096, d = 64, bf16), in its launch configuration (all 96 slices in one
    pass over the pair buffers, which the pair kernels take 16 at a time); the
    gradients of the first, a middle and the last slice against the oracle,
    slice by slice."""
    pa = _pa()
    wl = workloads.CONFIGS["lm"]
    x = workloads.make_inputs(wl, device=DEV, variant=3)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    do = torch.randn(x["q"].shape, generator=gen, device=DEV).to(wl.dtype)
    print(f"case bwd full lm {tuple(x['q'].shape)}", flush=True)
    o, lse = pa.fwd(x["q"], x["k"], x["v"], x["w"], x["beta"], logf=None, scale=wl.scale)
    grads = pa.bwd(x["q"], x["k"], x["v"], x["w"], x["beta"], None, o, lse, do, scale=wl.scale)
    torch.cuda.synchronize()
    nsl = wl.N * wl.H
    for s in (0, nsl // 2, nsl - 1):
        f64 = {k: (workloads.as_slices_f64(v, heads=[s]) if v is not None else None)
               for k, v in x.items()}
        ref = oracle.bwd(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], None, wl.scale,
                         workloads.as_slices_f64(do, heads=[s]))
        for name, got in zip(NAMES, grads):
            if ref[name] is None:
                continue
            ma, mr, gmax = _errs(workloads.as_slices_f64(got, heads=[s]), ref[name])
            msg = f"  slice {s} {name}: max-err/g_max {ma:.2e} mean-rel {mr:.2e} (g_max {gmax:.3g})"
            print(msg, flush=True)
            assert ma <= 2e-2 and mr <= 1e-2, msg
