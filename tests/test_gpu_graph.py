"""The training step (block forward with checkpoints, then block backward) captured
into a HIP graph through torch and replayed.  Every replay must equal the eager
step up to the look-back's rounding; eager calls and synchronisations run between
the replays, and the outputs are cleared before each one, so a replay that wrote
nothing would fail."""
import pytest
import torch

from gpu_helpers import assert_agree, dev, f32_dev, host, to_dev
from selective_state_space_naju_amd import binding as nb
from selective_state_space_naju_amd import inputs

pytestmark = pytest.mark.gpu


def test_block_step_graph_replays_match_eager():
    Bt, L, Di, N = 2, 1000, 256, 16
    print("graph step", Bt, L, Di, N, flush=True)
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=31, block=True, backward=True)
    t = {k: to_dev(d[k], "bf16") for k in ("u", "z", "a", "b", "B", "C", "dy")}
    D, cw = f32_dev(d["D"]), f32_dev(d["conv_w"])
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16)
    ws_f = nb.Workspace(nb.workspace_bytes(nb.OP_BLOCK_FWD, dims), dev())
    ws_b = nb.Workspace(nb.workspace_bytes(nb.OP_BLOCK_BWD, dims), dev())

    def step():
        y, xf, _, ck = nb.block_fwd(t["u"], t["z"], cw, t["a"], t["b"], t["B"], t["C"], D,
                                    return_ckpt=True, ws=ws_f)
        g = nb.block_bwd(t["u"], t["z"], cw, t["a"], t["b"], t["B"], t["C"], D, t["dy"],
                         ckpt=ck, ws=ws_b)
        return {k: v for k, v in dict(g, y=y, xf=xf).items() if v is not None}

    eager = {k: host(v) for k, v in step().items()}
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        out = step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert_agree("%s(replay %d)" % (k, rep), host(v), eager[k], ulps=2.0)
        step()  # eager work on the same workspaces between replays
        torch.cuda.synchronize()
    assert ws_f.error_flags() == 0 and ws_b.error_flags() == 0
