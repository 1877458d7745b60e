"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}  # relative error bound per io type


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
    if (np.isnan(got) != np.isnan(ref)).any():
        return np.inf
    m = ~(np.isnan(got) | np.isnan(ref))
    den = np.abs(ref[m]).max() if m.any() else 0.0
    num = np.abs(got[m] - ref[m]).max() if m.any() else 0.0
    return num / den if den > 0 else num


def elementwise(got, ref, tol):
    """Elementwise view of the error: the bound |got - ref| <= tol |ref| + atol with
    atol = tol * rms(ref) (the scale of the tensor's own rounding), the worst element
    against that bound, its own relative error, and the relative L2 error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~(np.isnan(got) | np.isnan(ref))
    g, r = got[m], ref[m]
    if r.size == 0:
        return {"ratio": 0.0, "worst": None, "rel_l2": 0.0}
    rms = float(np.sqrt(np.mean(r * r)))
    atol = tol * rms if rms > 0 else tol
    err = np.abs(g - r)
    ratio = err / (tol * np.abs(r) + atol)
    k = int(np.argmax(ratio))
    flat = np.flatnonzero(m.ravel())[k]
    idx = np.unravel_index(flat, ref.shape)
    nref = float(np.sqrt(np.sum(r * r)))
    return {"ratio": float(ratio[k]),
            "worst": (tuple(int(i) for i in idx), float(g[k]), float(r[k]),
                      float(err[k] / abs(r[k])) if r[k] != 0 else float("inf")),
            "rel_l2": float(np.sqrt(np.sum(err * err)) / nref) if nref > 0 else float(
                np.sqrt(np.sum(err * err)))}


def assert_close(name, got, ref, tol):
    """Both bounds: the normwise one (max|err| / max|ref| <= tol) and the elementwise
    one (|err| <= tol |ref| + tol rms(ref) at every element)."""
    e = rel_err(got, ref)
    el = elementwise(got, ref, tol) if np.isfinite(e) else {"ratio": np.inf, "worst": None,
                                                            "rel_l2": np.inf}
    w = el["worst"]
    wtxt = ("worst %s got %.6g ref %.6g (own rel %.2e)" % w) if w else ""
    print("  %-12s rel_err=%.3e rel_l2=%.3e elem=%.3f (tol %.0e) %s"
          % (name, e, el["rel_l2"], el["ratio"], tol, wtxt), flush=True)
    assert e <= tol, "%s: normwise relative error %.3e > %.0e" % (name, e, tol)
    assert el["ratio"] <= 1.0, ("%s: elementwise bound exceeded by %.3fx at %s"
                                % (name, el["ratio"], wtxt))


def assert_agree(name, got, ref, ulps=1.0, rtol_rms=1e-4):
    """Two GPU results that may differ only by rounding inside the kernels (a
    look-back folding a predecessor's aggregate instead of reading its inclusive
    state; a split of the sequence that moves the chunk boundaries): per element,
    within `ulps` bf16 spacings of the larger magnitude plus rtol_rms * rms(ref).
    The second term is the absolute scale of that rounding, which a near-zero
    output does not shrink: the matrix-core products carry bf16 hi + lo operands
    (about 2^-16 relative each), summed over a chunk's 32 tokens."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.maximum(np.abs(got), np.abs(ref))
    spacing = np.exp2(np.floor(np.log2(np.where(m > 0, m, 1.0))) - 7)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = ulps * spacing + rtol_rms * rms
    ratio = np.abs(got - ref) / bound
    k = int(np.argmax(ratio)) if ratio.size else 0
    worst = np.unravel_index(k, ref.shape) if ratio.size else ()
    r = float(ratio.max()) if ratio.size else 0.0
    print("  %-12s agree ratio=%.3f worst %s got %.6g ref %.6g" % (
        name, r, tuple(int(i) for i in worst), got[worst] if ratio.size else 0.0,
        ref[worst] if ratio.size else 0.0), flush=True)
    assert r <= 1.0, "%s: results differ beyond rounding (%.3fx the bound at %s)" % (
        name, r, tuple(int(i) for i in worst))
