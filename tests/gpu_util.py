"""Helpers for GPU parity tests: tolerances and comparisons against the oracle."""
import sys

import numpy as np
import torch

# bf16 storage with fp32 accumulation: relative L2 <= 1e-2 and max-abs <= 3e-2;
# fp32 storage and arithmetic: both <= 1e-5.
TOL = {torch.bfloat16: (1e-2, 3e-2), torch.float32: (1e-5, 1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    diff = got - want
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300))
    return rel, float(np.abs(diff).max())


def assert_close(got, want, dtype, what=""):
    rel_tol, abs_tol = TOL[dtype]
    rel, mx = errors(got, want)
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e} (tol {rel_tol:g}, {abs_tol:g})")
    assert np.isfinite(rel) and np.isfinite(mx), what
    assert rel <= rel_tol and mx <= abs_tol, f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e}"


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def guarded_empty(shape, dtype, device, guard=4096):
    """An output tensor followed by a NaN-filled guard band (catches stray writes)."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), float("nan"), dtype=dtype, device=device)
    return buf, buf[:n].view(shape)


def guard_intact(buf, shape):
    n = int(np.prod(shape))
    return bool(torch.isnan(buf[n:]).all().item())
