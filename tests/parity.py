"""Tolerance checks shared by the GPU parity tests.

Floating-point bars (fixed by the workload definitions):
  float32 inputs: max-abs <= 1e-4 on o and lse;
  bf16 inputs:    max-abs <= 2e-2 and mean-rel <= 5e-3 on o and on lse,
against the fp64 oracle fed the same (bf16-rounded) inputs.
mean-rel = sum |got - ref| / sum |ref| over the checked elements.
"""
import numpy as np

F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 5e-3


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.abs(got - ref)
    return float(err.max()), float(err.sum() / max(np.abs(ref).sum(), 1e-300))


def check(name, got, ref, bf16: bool):
    ma, mr = errors(got, ref)
    if bf16:
        ok = ma <= BF16_MAX_ABS and mr <= BF16_MEAN_REL
        bar = f"max-abs<={BF16_MAX_ABS}, mean-rel<={BF16_MEAN_REL}"
    else:
        ok = ma <= F32_MAX_ABS
        bar = f"max-abs<={F32_MAX_ABS}"
    msg = f"{name}: max-abs {ma:.3e} mean-rel {mr:.3e} ({bar})"
    print(msg, flush=True)
    assert ok, msg
    return ma, mr


def cache_bar(k_dtype, rewrites: int):
    """Bar for the rewritten key cache, derived from its arithmetic (no stated
    tolerance applies to this internal state).  Every rewrite stores the key
    rounded to k_dtype, relative error <= u (u = 2^-9 for bf16, 2^-24 for
    fp32), and independent roundings add up like a random walk over the
    rewrites a key has seen; the prefill alignment contributes one more
    rounding of a product computed in fp32 (for fp32 caches u is taken as
    64 ulp to cover that product's accumulation).  Bars:
    mean-rel <= 2u (1 + sqrt(r)), max-abs <= 8u (1 + sqrt(r)) max|ref|."""
    import torch
    u = 2.0 ** -9 if k_dtype == torch.bfloat16 else 2.0 ** -24 * 64
    walk = 1 + rewrites ** 0.5
    return 2 * u * walk, 8 * u * walk


def check_cache(name, got, ref, k_dtype, rewrites):
    mr_bar, ma_rel = cache_bar(k_dtype, rewrites)
    ma_bar = ma_rel * float(np.abs(ref).max())
    ma, mr = errors(got, ref)
    msg = f"{name}: max-abs {ma:.3e} mean-rel {mr:.3e} (max-abs<={ma_bar}, mean-rel<={mr_bar:.3e})"
    print(msg, flush=True)
    assert ma <= ma_bar and mr <= mr_bar, msg
    return ma, mr
