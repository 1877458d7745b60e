"""The allocation-free scan forward (naju_scan_fwd_noalloc) against the workspace
entry point naju_scan_fwd, through the C ABI: two calls in a row on the same
GPU (the second smaller, so the shared scratch is reused with another layout),
both io types, checked to the parity bar (and against each other to rounding)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, assert_agree, assert_close, f32_dev, host, to_dev
from selective_state_space_naju_amd import binding as nb
from selective_state_space_naju_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    nb.lib()


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _both(Bt, L, Di, N, io, seed):
    d = inputs.draw(Bt, L, Di, N, io=io, seed=seed, x0=True)
    t = {k: to_dev(d[k], io) for k in ("h", "a", "b", "B", "C")}
    D, x0 = f32_dev(d["D"]), f32_dev(d["x0"])
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16 if io == "bf16" else nb.F32)
    L_ = nb.lib()
    y0, y1 = (torch.empty((Bt, L, Di), dtype=dt, device="cuda") for _ in range(2))
    x_0, x_1 = (torch.empty((Bt, Di, N), dtype=torch.float32, device="cuda") for _ in range(2))
    ws = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, dims), torch.device("cuda"))
    nb.check(L_.naju_scan_fwd(ctypes.byref(dims), _p(t["h"]), _p(t["a"]), _p(t["b"]),
                              _p(t["B"]), _p(t["C"]), _p(D), _p(x0), _p(y0), _p(x_0), None,
                              ws.ptr, ws.nbytes, nb.stream_handle()))
    flags = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    nb.check(L_.naju_scan_fwd_noalloc(ctypes.byref(dims), _p(t["h"]), _p(t["a"]), _p(t["b"]),
                                      _p(t["B"]), _p(t["C"]), _p(D), _p(x0), _p(y1), _p(x_1),
                                      None, _p(flags), nb.stream_handle()))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert ws.error_flags() == 0
    return host(y0), host(x_0), host(y1), host(x_1)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(io):
    for (Bt, L, Di, N, seed) in ((4, 2100, 264, 16, 41), (2, 300, 200, 16, 42)):
        print("no-alloc", io, Bt, L, Di, N, flush=True)
        y0, xf0, y1, xf1 = _both(Bt, L, Di, N, io, seed)
        assert_close("y", y1, y0, TOL[io])
        assert_close("x_final", xf1, xf0, TOL[io])
        if io == "bf16":
            assert_agree("y(agree)", y1, y0)
        else:
            assert np.abs(y1 - y0).max() <= 1e-5 * np.abs(y0).max()
        assert np.abs(xf1 - xf0).max() <= 1e-5 * np.abs(xf0).max()
