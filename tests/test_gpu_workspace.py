"""Workspace hygiene on the GPU, through the C ABI: no entry point may depend on what its
workspace held before the call. Each call runs on a workspace filled with 0x00, 0xFF (NaN as
floats, -1 as ints) and 0x7F bytes; the outputs, NaN-poisoned beforehand, must come back finite
and bitwise equal across the three fills."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from tests.test_gpu_parity import SMALL, _shape

pytestmark = pytest.mark.gpu

FILLS = (0x00, 0xFF, 0x7F)


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _ws(nbytes, fill):
    return torch.full((max(1, nbytes),), fill, dtype=torch.uint8, device="cuda")


def _same(outs):
    ref = outs[0]
    for o in outs:
        assert np.isfinite(o).all()
        assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name,layout", [("tiny", 0), ("mid_T2000", 0), ("mid_conc_T64", 1), ("beam1", 1),
                                         ("beam2", 1)])
def test_forward_ignores_workspace_contents(name, layout):
    w = recipes.WORKLOADS[int(name[4:])] if name.startswith("beam") else SMALL[name]
    print("case workspace forward", name, layout, flush=True)
    t = synth.device_inputs(w)
    shape = moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob, w.eps,
                           weight_layout=layout)
    W = moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]) if layout else (t["Wg"], t["Wu"], t["Wd"])
    hid = t["h"] if w.prenorm else t["x"]
    ys, ws_ = [], []
    for f in FILLS:
        ws = _ws(moe.beam_moe_workspace_bytes(shape), f)
        y = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((w.T, w.top_k), -7, dtype=torch.int32, device="cuda")
        wt = torch.full((w.T, w.top_k), float("nan"), dtype=torch.float32, device="cuda")
        moe.beam_moe_forward(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], *W, y, idx, wt, None, ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
        ws_.append((idx.cpu().numpy(), wt.cpu().numpy()))
    _same(ys)
    for idx, wt in ws_:
        assert np.array_equal(idx, ws_[0][0]) and np.array_equal(wt.view(np.uint32), ws_[0][1].view(np.uint32))


def test_share_and_dense_ignore_workspace_contents():
    w = SMALL["mid_T77"]
    t = synth.device_inputs(w)
    shape = _shape(w)
    ws = _ws(moe.beam_moe_workspace_bytes(shape), 0)
    y = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    moe.beam_moe_forward(shape, t["x"], None, t["Wr"], t["bias"], t["Wg"], t["Wu"], t["Wd"], y, idx, wt, None, ws)
    e0, n = 64, 32
    outs = []
    for f in FILLS:
        sws = _ws(moe.beam_moe_share_workspace_bytes(shape, n), f)
        yp = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
        moe.beam_moe_experts_share(shape, e0, n, t["x"], idx, wt, t["Wg"][e0:e0 + n], t["Wu"][e0:e0 + n],
                                   t["Wd"][e0:e0 + n], yp, sws)
        torch.cuda.synchronize()
        outs.append(yp.cpu().numpy())
    _same(outs)
    for T in (33, 300):                    # the dense decode streams and the dense GEMM
        dw = recipes.DENSE_WORKLOADS[12].with_T(T)
        dt = synth.dense_device_inputs(dw)
        outs = []
        for f in FILLS:
            dws = _ws(moe.beam_moe_dense_workspace_bytes(dw.T, dw.d, dw.I), f)
            yd = torch.full((dw.T, dw.d), float("nan"), dtype=torch.float32, device="cuda")
            moe.beam_moe_dense_mlp(dw.T, dw.d, dw.I, dt["x"], dt["Wg"], dt["Wu"], dt["Wd"], yd, dws)
            torch.cuda.synchronize()
            outs.append(yd.cpu().numpy())
        _same(outs)


def test_two_layers_on_two_streams_at_once():
    """No state outside the caller's workspace: two layers (weight streams and tiled GEMM paths)
    launched concurrently on two streams, with their own workspaces, give the same bits as each
    run alone."""
    cases = []
    for name, layout in (("mid_T77", 1), ("mid_T2000", 1)):
        w = SMALL[name]
        t = synth.device_inputs(w)
        shape = moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob,
                               w.eps, weight_layout=layout)
        W = moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]) if layout else (t["Wg"], t["Wu"], t["Wd"])
        ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        y = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
        hid = t["h"] if w.prenorm else t["x"]
        cases.append(((shape, hid, t.get("norm_w"), t["Wr"], t["bias"], *W, y, None, None, None, ws), y, t))
    alone = []
    for args, y, _ in cases:
        moe.beam_moe_forward(*args)
        torch.cuda.synchronize()
        alone.append(y.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for _, y, _ in cases:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        for (args, _, _), st in zip(cases, streams):
            moe.beam_moe_forward(*args, stream=st.cuda_stream)
        torch.cuda.synchronize()
        for (_, y, _), ref in zip(cases, alone):
            assert torch.equal(y, ref), "concurrent run %d differs" % rep
