"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}  # normwise relative error bound per io type


def dev():
    return torch.device("cuda:0")


def to_dev(x, io, device=None):
    """float32 numpy (values already representable in the io type) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device or dev())


def f32_dev(x, device=None):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device or dev())


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max |got - ref| / max |ref| (normwise infinity), with NaN treated as a failure."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError("shape %s vs %s" % (got.shape, ref.shape))
    if got.size == 0:
        return 0.0
    if np.isnan(got).any() != np.isnan(ref).any():
        return np.inf
    m = ~(np.isnan(got) | np.isnan(ref))
    den = np.abs(ref[m]).max() if m.any() else 0.0
    num = np.abs(got[m] - ref[m]).max() if m.any() else 0.0
    return num / den if den > 0 else num


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    print("  %-12s rel_err=%.3e (tol %.0e)" % (name, e, tol), flush=True)
    assert e <= tol, "%s: normwise relative error %.3e > %.0e" % (name, e, tol)
