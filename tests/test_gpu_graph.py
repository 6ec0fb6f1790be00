"""The layer under HIP graph capture (torch.cuda.CUDAGraph, which is a hipGraph on ROCm): the
C ABI allocates nothing, synchronises nothing and writes no memsets, so a captured call replays.
Each replay runs with eager work of other shapes in between and must give the eager result bit
for bit (a replay that reused stale state from an earlier one would differ)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from tests.test_gpu_parity import SMALL
from tests.test_gpu_packed import WS_CASES

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _setup(w, layout):
    t = synth.device_inputs(w)
    shape = moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob, w.eps,
                           weight_layout=layout)
    W = moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]) if layout else (t["Wg"], t["Wu"], t["Wd"])
    ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    hid = t["h"] if w.prenorm else t["x"]
    args = (shape, hid, t.get("norm_w"), t["Wr"], t["bias"], *W, y, idx, wt, None, ws)
    return t, args, y


# mid_T2100 (packed): the gate/up GEMM on the persistent weight-streaming kernel; ws_mid_T1500
# (packed, d = I = 512): both expert GEMMs on it, their work-item counters cleared inside the graph
@pytest.mark.parametrize("name,layout", [("beam1", 1), ("mid_T2000", 0), ("mid_T2100", 1), ("mid_prenorm_T333", 1),
                                         ("ws_mid_T1500", 1)])
def test_graph_replay_matches_eager(name, layout):
    w = recipes.WORKLOADS[1] if name == "beam1" else (WS_CASES[name] if name in WS_CASES else SMALL[name])
    print("case graph", name, layout, flush=True)
    t, args, y = _setup(w, layout)
    moe.beam_moe_forward(*args)
    torch.cuda.synchronize()
    eager = y.clone()
    # other work in between replays: a different layer with its own buffers
    o = SMALL["mid_T77"]
    _, oargs, oy = _setup(o, 0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up on the capture stream, as torch asks
        moe.beam_moe_forward(*args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    y.fill_(float("nan"))
    with torch.cuda.graph(g):
        moe.beam_moe_forward(*args)
    for rep in range(3):
        y.fill_(float("nan"))
        moe.beam_moe_forward(*oargs)           # eager work on other buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), "replay %d differs from the eager call" % rep
    assert np.isfinite(oy.cpu().numpy()).all()
