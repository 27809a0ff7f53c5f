"""The method's exact special cases run through the PaTH kernels on the GPU
(reading-notes page "PaTH Attention:通过累积 Householder 变换编码位置"):

* beta = 0 makes every transition the identity (s2.1, s2.2), so PaTH is
  plain causal softmax attention (with the gate: forgetting attention, s2.5):
  checked against the oracle and against the library's own causal kernel;
* beta = 2 makes every transition a reflection (s2.2), the far end of the
  range, where the block transitions do not contract the carried queries;
* the path of key j to query i uses H_{j+1} ... H_i only (s2.1), so w_0 and
  beta_0 never reach any output: changing them must leave o, lse and the
  aligned decode cache bit for bit unchanged.  log f_0 never reaches an
  output either, but the kernels add gate prefixes that include it and
  subtract them again, so there the check is against the oracle's bar.
"""
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


def _with_beta(x, value):
    y = dict(x)
    y["beta"] = torch.full_like(x["beta"], float(value))
    return y


def _fwd_vs_oracle(name, wl, x, cache=None, rows=None):
    pa = _pa()
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    print(f"case {name} {tuple(x['q'].shape)} {wl.dtype}", flush=True)
    o, lse = pa.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"], scale=wl.scale,
                    cache=cache)
    torch.cuda.synchronize()
    f64 = {k: (workloads.as_slices_f64(v) if v is not None else None) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=rows)
    go, gl = workloads.as_slices_f64(o), workloads.as_slices_f64(lse)
    if rows is not None:
        go, gl = go[:, rows], gl[:, rows]
    bf = wl.dtype == torch.bfloat16
    check(f"{name} o", go, ro, bf16=bf)
    check(f"{name} lse", gl, rl, bf16=bf)
    return o, lse, g


@pytest.mark.parametrize("fox", [False, True])
def test_beta_zero_bf16_is_causal_attention(fox):
    """beta = 0 through path_attn_fwd (bf16, d = 64, ragged L): equal to the
    oracle, and without the gate equal to the causal baseline kernel up to
    the order of fp32 accumulation (both round o to bf16)."""
    wl = workloads.CONFIGS["lm"].replace(N=2, H=3, L=1000, fox=fox)
    x = _with_beta(workloads.make_inputs(wl, L=wl.L), 0.0)
    o, lse, g = _fwd_vs_oracle(f"beta=0 bf16 fox={fox}", wl, x)
    if not fox:
        # The two kernels round the probabilities to bf16 against their own
        # running maxima (and sum those rounded values into lse), so they
        # agree to the bf16 bar, not bit for bit.
        co, cl = _pa().causal_attn(g["q"], g["k"], g["v"], scale=wl.scale)
        torch.cuda.synchronize()
        check("beta=0 PaTH vs causal kernel o", o.float().cpu().numpy(), co.float().cpu().numpy(),
              bf16=True)
        check("beta=0 PaTH vs causal kernel lse", lse.cpu().numpy(), cl.cpu().numpy(), bf16=True)


@pytest.mark.parametrize("d", [16, 64])
def test_beta_zero_fp32(d):
    wl = workloads.CONFIGS["tiny"].replace(H=3, d=d, L=150, fox=True, scale=d ** -0.5)
    _fwd_vs_oracle(f"beta=0 fp32 d={d}", wl, _with_beta(workloads.make_inputs(wl, L=wl.L), 0.0))


@pytest.mark.parametrize("fox", [False, True])
@pytest.mark.parametrize("d", [16, 32])
def test_beta_two_fp32(d, fox):
    wl = workloads.CONFIGS["tiny"].replace(H=2, d=d, L=300, fox=fox, scale=d ** -0.5)
    _fwd_vs_oracle(f"beta=2 fp32 d={d} fox={fox}", wl,
                   _with_beta(workloads.make_inputs(wl, L=wl.L), 2.0))


def test_beta_two_bf16_fox():
    """Reflections everywhere with the forget gate, as in the long-context
    workload (bf16, d = 64, ragged L, several blocks)."""
    wl = workloads.CONFIGS["fox"].replace(N=1, H=4, L=1000)
    _fwd_vs_oracle("beta=2 bf16 fox", wl, _with_beta(workloads.make_inputs(wl, L=wl.L), 2.0))


def test_beta_two_bf16_no_gate_short():
    """Reflections without the gate over four blocks (d = 32 and 64)."""
    for d in (32, 64):
        wl = workloads.CONFIGS["lm"].replace(N=1, H=4, L=256, d=d, qk_std=d ** -0.25)
        _fwd_vs_oracle(f"beta=2 bf16 no gate d={d}", wl,
                       _with_beta(workloads.make_inputs(wl, L=wl.L), 2.0))


@pytest.mark.parametrize("dtype,k_dtype", [(torch.bfloat16, torch.float32),
                                           (torch.bfloat16, torch.bfloat16),
                                           (torch.float32, torch.float32)])
def test_beta_two_decode(dtype, k_dtype):
    """Prefill with cache alignment and fused decode steps with every beta = 2
    (and the gate): decode outputs against the oracle's rows, the final cache
    against the explicitly transported keys."""
    pa = _pa()
    wl = workloads.CONFIGS["fox"].replace(N=1, H=3, L=330, dtype=dtype)
    steps = 10
    x = _with_beta(workloads.make_inputs(wl, L=wl.L + steps), 2.0)
    g = {k: v.to(DEV) for k, v in x.items()}
    L = wl.L
    print(f"case beta=2 decode {dtype} keys {k_dtype}", flush=True)
    cache = pa.Cache(1, wl.H, L + steps, wl.d, dtype=dtype, k_dtype=k_dtype, gate=True,
                     device=DEV)
    pre = lambda n: g[n][:, :, :L].contiguous()
    pa.fwd(pre("q"), pre("k"), pre("v"), pre("w"), pre("beta"), logf=pre("logf"),
           scale=wl.scale, cache=cache)
    tok = lambda n, t: g[n][:, :, t].contiguous()
    outs = [pa.decode_step(cache, t, *(tok(n, t) for n in ("q", "k", "v", "w", "beta", "logf")),
                           scale=wl.scale) for t in range(L, L + steps)]
    torch.cuda.synchronize()
    f64 = {k: workloads.as_slices_f64(v) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=np.arange(L, L + steps))
    bf = dtype == torch.bfloat16
    check("beta=2 decode o", np.stack([workloads.as_slices_f64(o) for o, _ in outs], 1), ro, bf)
    check("beta=2 decode lse", np.stack([workloads.as_slices_f64(l) for _, l in outs], 1), rl, bf)
    rk = oracle.transported_keys(f64["k"], f64["w"], f64["beta"], L + steps - 1)
    check_cache("beta=2 kcache", workloads.as_slices_f64(cache.kcache), rk, k_dtype, steps)


def _prefill_with_cache(x, wl):
    pa = _pa()
    g = {k: v.to(DEV) for k, v in x.items()}
    N, H, L, d = g["q"].shape
    cache = pa.Cache(N, H, L, d, dtype=wl.dtype, gate=g["logf"] is not None, device=DEV)
    o, lse = pa.fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], logf=g["logf"], scale=wl.scale,
                    cache=cache)
    torch.cuda.synchronize()
    return o, lse, cache


@pytest.mark.parametrize("cfg,dtype,d", [("fox", torch.bfloat16, 64), ("flipflop", torch.bfloat16, 32),
                                         ("tiny", torch.float32, 16), ("tiny", torch.float32, 64)])
def test_first_transition_never_matters(cfg, dtype, d):
    """w_0 and beta_0 are on no path (H_j is excluded from key j's path and
    key 0 is the first), so changing them leaves o, lse and the aligned cache
    bit-identical; the gate's log f_0 is checked against the oracle."""
    wl = workloads.CONFIGS[cfg].replace(N=2, H=2, L=300, d=d, dtype=dtype, fox=True)
    x = workloads.make_inputs(wl, L=wl.L)
    print(f"case first transition {cfg} {dtype} d={d}", flush=True)
    o0, l0, c0 = _prefill_with_cache(x, wl)
    for beta0 in (0.0, 2.0, 0.37):
        y = dict(x)
        y["beta"] = x["beta"].clone()
        y["beta"][:, :, 0] = beta0
        w = x["w"].clone().float()
        w[:, :, 0] = torch.flip(w[:, :, 0], dims=[-1]) * -1.0       # another unit vector
        y["w"] = w.to(dtype)
        o1, l1, c1 = _prefill_with_cache(y, wl)
        assert torch.equal(o0, o1), f"o depends on w_0/beta_0 (beta_0 = {beta0})"
        assert torch.equal(l0, l1), f"lse depends on w_0/beta_0 (beta_0 = {beta0})"
        assert torch.equal(c0.kcache, c1.kcache), "cached keys depend on w_0/beta_0"
        assert torch.equal(c0.vcache, c1.vcache) and torch.equal(c0.gcache, c1.gcache)
    # log f_0 far outside its usual range: the kernels' block-relative gate
    # sums carry it and cancel it, so the result must still meet the bar
    # against the oracle (which never reads log f_0)
    y = dict(x)
    y["logf"] = x["logf"].clone()
    y["logf"][:, :, 0] = -7.5
    o2, l2, _ = _prefill_with_cache(y, wl)
    f64 = {k: workloads.as_slices_f64(v) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale)
    bf = dtype == torch.bfloat16
    check("log f_0 = -7.5 o", workloads.as_slices_f64(o2), ro, bf16=bf)
    check("log f_0 = -7.5 lse", workloads.as_slices_f64(l2), rl, bf16=bf)
