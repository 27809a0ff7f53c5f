"""The allocation-free fused decode step (path_decode_step_noalloc), called
through the C ABI, against path_decode_step with a caller workspace: the same
kernels, so the outputs and the rewritten cache must agree bit for bit, and
both meet the oracle's bar.  Two calls in a row, the second smaller (fewer
slices and keys) than the first, so the shared device scratch holds the first
call's larger contents when the second runs."""
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


def _prefilled(pa, wl, x, L, cap, k_dtype):
    c = pa.Cache(wl.N, wl.H, cap, wl.d, dtype=wl.dtype, k_dtype=k_dtype, gate=True, device=DEV)
    pre = lambda n: x[n][:, :, :L].contiguous()
    pa.fwd(pre("q"), pre("k"), pre("v"), pre("w"), pre("beta"), logf=pre("logf"),
           scale=wl.scale, cache=c)
    return c


def _case(wl, L, steps, k_dtype):
    pa = _pa()
    x = {k: v.to(DEV) for k, v in workloads.make_inputs(wl, L=L + steps).items()}
    print(f"case noalloc N={wl.N} H={wl.H} L={L} steps={steps} keys {k_dtype}", flush=True)
    a = _prefilled(pa, wl, x, L, L + steps, k_dtype)
    b = _prefilled(pa, wl, x, L, L + steps, k_dtype)
    got = []
    for t in range(L, L + steps):
        tok = [x[n][:, :, t].contiguous() for n in ("q", "k", "v", "w", "beta", "logf")]
        ro, rl = pa.decode_step(a, t, *tok, scale=wl.scale)
        o, lse = pa.decode_step_noalloc(b, t, *tok, scale=wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(lse, rl), f"step {t} differs"
        got.append((o, lse))
    assert torch.equal(a.kcache, b.kcache) and torch.equal(a.vcache, b.vcache)
    assert torch.equal(a.gcache, b.gcache)
    f64 = {k: workloads.as_slices_f64(v) for k, v in x.items()}
    ro, rl = oracle.fwd_rows(f64["q"], f64["k"], f64["v"], f64["w"], f64["beta"], f64["logf"],
                             wl.scale, rows=np.arange(L, L + steps))
    bf = wl.dtype == torch.bfloat16
    check("noalloc o", np.stack([workloads.as_slices_f64(o) for o, _ in got], 1), ro, bf)
    check("noalloc lse", np.stack([workloads.as_slices_f64(l) for _, l in got], 1), rl, bf)
    rk = oracle.transported_keys(f64["k"], f64["w"], f64["beta"], L + steps - 1)
    check_cache("noalloc kcache", workloads.as_slices_f64(b.kcache), rk, k_dtype, steps)


def test_noalloc_step_matches_workspace_step_twice():
    # first call: 32 slices x 5001 keys; second: 3 slices x 301 keys, fp32 keys
    _case(workloads.CONFIGS["fox"].replace(N=2, H=16), 5000, 2, torch.bfloat16)
    _case(workloads.CONFIGS["fox"].replace(N=1, H=3, dtype=torch.float32), 300, 2, torch.float32)

