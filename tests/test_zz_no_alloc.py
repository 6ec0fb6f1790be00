"""beam_moe_forward_noalloc (the layer on the library's fixed per-GPU scratch, for callers that
cannot allocate) against beam_moe_forward with a caller workspace, through the C ABI: two calls in
a row at the Beam decode shape, the second with fewer tokens, each bitwise equal to the workspace
entry point (same kernels, same arithmetic), on packed and on row-major expert weights."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes

pytestmark = pytest.mark.gpu


def _outputs(w, dev):
    return dict(y=torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device=dev),
                idx=torch.full((w.T, w.top_k), -7, dtype=torch.int32, device=dev),
                wt=torch.full((w.T, w.top_k), float("nan"), dtype=torch.float32, device=dev),
                z=torch.full((w.T, w.E), float("nan"), dtype=torch.float32, device=dev))


def _same(a, b):
    return np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("layout", ["packed", "row-major"])
def test_noalloc_matches_workspace_entry_point(layout):
    dev = torch.device("cuda")
    full = recipes.WORKLOADS[1].with_T(192)
    print("case noalloc", layout, flush=True)
    t = synth.device_inputs(full)
    W = moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]) if layout == "packed" else (t["Wg"], t["Wu"], t["Wd"])
    lay = moe.WEIGHTS_PACKED if layout == "packed" else moe.WEIGHTS_ROW_MAJOR
    for T in (192, 64):                     # the largest batch the scratch takes, then a smaller one
        w = full.with_T(T)
        shape = moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob,
                               w.eps, weight_layout=lay)
        x = t["x"][:T]
        ref = _outputs(w, dev)
        ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        moe.beam_moe_forward(shape, x, None, t["Wr"], t["bias"], *W, ref["y"], ref["idx"], ref["wt"], ref["z"], ws)
        got = _outputs(w, dev)
        moe.beam_moe_forward_noalloc(shape, x, None, t["Wr"], t["bias"], *W, got["y"], got["idx"], got["wt"],
                                     got["z"])
        torch.cuda.synchronize()
        print("T=%d: compared y, idx, w, logits" % T, flush=True)
        assert torch.isfinite(got["y"]).all()
        for k in ("y", "idx", "wt", "z"):
            assert _same(got[k], ref[k]), "T=%d: %s differs from beam_moe_forward" % (T, k)
        del ws
