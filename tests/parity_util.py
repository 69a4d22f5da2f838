"""Shared helpers of the parity tests (tolerance checks, device transfer)."""
import numpy as np
import torch

# Tolerances: bf16 inputs with fp32 accumulation |g - r| <= 2e-2 + 1e-2 |r|;
# the fp32 path 1e-4 + 1e-4 |r|; scores 5e-3 absolute.
BF16_TOL = (2e-2, 1e-2)
F32_TOL = (1e-4, 1e-4)
SCORE_ATOL = 5e-3


def assert_close(got, ref, atol, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    ok = np.abs(got - ref) <= atol + rtol * np.abs(ref)   # NaN -> not ok
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)}/{ok.size} elements out of tolerance (atol={atol}, rtol={rtol}); "
            f"first at {i}: got {got[i]!r} ref {ref[i]!r}; max|d|={np.nanmax(np.abs(got - ref)):.3e}")


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy() if t.dtype.is_floating_point else t.cpu().numpy()


def stack_tol(dtype):
    return F32_TOL if dtype == "f32" else BF16_TOL
