"""GPU parity of the parameter front-end (path_param_fwd) against the fp64
oracle on the same rounded inputs: w in the output dtype's bar (bf16: max-abs
2e-2 and mean-rel 5e-3; fp32: max-abs 1e-4), beta and log f (float32
outputs computed in fp32) at max-abs 1e-4."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import check

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(N, L, Dm, R, H, d, dtype, gate, seed=0):
    import dependent_position_encoding_amd as pa
    pa.load_library()
    print(f"case frontend N={N} L={L} Dm={Dm} R={R} H={H} d={d} {dtype} gate={gate}", flush=True)
    p = workloads.make_frontend_inputs(N, L, Dm, R, H, d, dtype, gate, device="cpu", seed=seed)
    g = {k: v.to(DEV) for k, v in p.items()}
    w, beta, logf = pa.param_fwd(**g, H=H, d=d)
    torch.cuda.synchronize()
    f64 = {k: v.to(torch.float64).numpy() for k, v in p.items()}
    rw, rb, rl = oracle.frontend(**f64, H=H, d=d)
    bf = dtype == torch.bfloat16
    check("frontend w", w.to(torch.float64).cpu().numpy().reshape(N * H, L, d),
          rw.reshape(N * H, L, d), bf16=bf)
    assert np.abs(beta.cpu().double().numpy() - rb).max() < 1e-4
    if gate:
        assert np.abs(logf.cpu().double().numpy() - rl).max() < 1e-4
    else:
        assert logf is None
    return w, beta, logf


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_frontend_small(dtype, d):
    # ragged L (not a multiple of the 32-token tile), rank 16, odd head count
    _run(2, 77, 64, 16, 3, d, dtype, gate=(d != 32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("R,Dm,H,d", [(48, 80, 5, 32), (96, 208, 9, 64)])
def test_frontend_ranks(dtype, R, Dm, H, d):
    # ranks past the register-held up-projection (48: four rank steps; 96:
    # loaded per step), an input width with a partial last chunk, head counts
    # that are not a multiple of the 4-head group or the 8-column padding, and
    # 150 tokens: a partial 128-token projection tile and 32-token finish tile
    _run(1, 150, Dm, R, H, d, dtype, gate=True, seed=2)


def test_frontend_lm_shape():
    # the LM-layer shape: 4 x 4096 tokens, 24 heads of 64 (width 1536), rank 32
    _run(4, 4096, 1536, 32, 24, 64, torch.bfloat16, gate=True, seed=1)


def test_frontend_first_tokens_and_zero_input():
    """The convolution is causal (token 0 sees only its own row) and an
    all-zero input row gives w = 0 and beta = 2 sigma(bb)."""
    import dependent_position_encoding_amd as pa
    p = workloads.make_frontend_inputs(1, 40, 32, 16, 2, 32, torch.float32, True, device=DEV)
    p["x"][:, 5:8] = 0.0       # three zero rows: c_7 = 0 exactly
    w, beta, logf = pa.param_fwd(**p, H=2, d=32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(w[:, :, 7]) == 0
    assert torch.allclose(beta[:, :, 7], 2 * torch.sigmoid(p["bb"])[None, :], atol=1e-6)
    f64 = {k: v.cpu().double().numpy() for k, v in p.items()}
    rw, _, _ = oracle.frontend(**f64, H=2, d=32)
    assert np.abs(w.cpu().double().numpy()[:, :, :3] - rw[:, :, :3]).max() < 1e-4
