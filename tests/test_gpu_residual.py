"""Post-MLP RMSNorm + depth-scaled FP32 residual on the GPU, through the C ABI, against
the oracle's post_norm / residual_step (double).

Two bars: on the GPU's own y the fused epilogue must agree with the oracle to FP32
rounding (the only difference is FP32 arithmetic against double); against the oracle's
y the error is the layer's y error carried through the norm, bounded from the y bar."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from synth.recipes import Workload
from tests import _parity as P
from tests.test_gpu_parity import SMALL, _eps32, _oracle_inputs, _experts_host, _shape

pytestmark = pytest.mark.gpu

# Per element: |gpu - oracle| <= REL * (|resid * keep| + |n * add|) + ABS. FP32 keeps 24 bits;
# the row's sum of squares over up to 16384 terms and the reciprocal square root each add a
# few units of rounding, far below this.
REL, ABS = 4e-6, 1e-30


def _factors(layer):
    k = oracle.contribution_index(layer, True)
    return np.sqrt((k - 1) / k), 1 / np.sqrt(k)


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def _check_tight(got, y, post_w, eps, resid, layer):
    ref = oracle.post_residual(y, post_w, eps, resid, layer)
    keep, add = _factors(layer)
    n = oracle.post_norm(y, post_w, eps)
    bound = REL * (np.abs(resid.astype(np.float64) * keep) + np.abs(n * add)) + ABS
    bad = np.abs(got.astype(np.float64) - ref) > bound
    assert not bad.any(), "%d elements off; worst %.3e" % (bad.sum(), np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("T,d,layer,scale", [(1, 64, 0, 1.0), (37, 192, 3, 0.05), (64, 5120, 3, 0.05),
                                             (300, 5120, 51, 30.0), (5, 16384, 10, 1e-3), (1500, 320, 7, 2.0)])
def test_post_residual_standalone(T, d, layer, scale):
    print("case post_residual T=%d d=%d layer=%d" % (T, d, layer), flush=True)
    w = Workload(40, "post_T%d_d%d" % (T, d), T=T, d=d, E=16, n_group=4, topk_group=2, top_k=4, I=64)
    rng = np.random.default_rng(T * 7 + d)
    y = (rng.standard_normal((T, d)) * scale).astype(np.float32)
    resid = synth.residual(w)
    pw = synth.post_norm_weight(w)
    shape = _shape(w)
    y_d, r_d, pw_d = _dev(y), _dev(resid), _dev(pw.view(np.int16), torch.bfloat16)
    out = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    moe.beam_moe_post_residual(shape, y_d, pw_d, layer, r_d, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    _check_tight(got, y.astype(np.float64), pw, _eps32(w), resid, layer)
    # in place: the same bits as out of place
    moe.beam_moe_post_residual(shape, y_d, pw_d, layer, r_d, r_d)
    torch.cuda.synchronize()
    assert np.array_equal(r_d.cpu().numpy(), got)


FUSED = {**{k: SMALL[k] for k in ("tiny", "mid_T77", "mid_T2000", "mid_prenorm_T333")},
         "beam_decode_T64": recipes.WORKLOADS[1], "beam_prefill_T8192": recipes.WORKLOADS[2]}


@pytest.mark.parametrize("name", list(FUSED))
def test_forward_residual(name):
    """Fused combine + post-norm + residual: y bitwise equal to beam_moe_forward's, the
    residual tight against the oracle on that y for every token, and within the carried
    y bar against the oracle's own layer output on a token sample."""
    w = FUSED[name]
    layer = 3 + (w.T % 40)
    print("case forward_residual", name, "layer", layer, flush=True)
    t = synth.device_inputs(w)
    shape = _shape(w)
    hid = t["h"] if w.prenorm else t["x"]
    ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    y0 = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.beam_moe_forward(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], t["Wg"], t["Wu"], t["Wd"], y0, idx, wt,
                         None, ws)
    resid = synth.residual(w)
    pw = synth.post_norm_weight(w)
    r_d, pw_d = _dev(resid), _dev(pw.view(np.int16), torch.bfloat16)
    out = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    y1 = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.beam_moe_forward_residual(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], t["Wg"], t["Wu"], t["Wd"], pw_d,
                                  layer, r_d, out, y1, None, None, None, ws)
    out2 = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.beam_moe_forward_residual(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], t["Wg"], t["Wu"], t["Wd"], pw_d,
                                  layer, r_d, out2, None, None, None, None, ws)
    torch.cuda.synchronize()
    y0, y1, got = y0.cpu().numpy(), y1.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(out2.cpu().numpy().view(np.uint32), got.view(np.uint32))
    eps = _eps32(w)
    _check_tight(got, y1.astype(np.float64), pw, eps, resid, layer)

    # against the oracle's own layer output on a sample of tokens
    x, Wr, b = _oracle_inputs(w)
    idx_ref, w_ref, gap, z_ref = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale,
                                              w.norm_topk_prob, want_logits=True)
    same = P.compare_routing(idx.cpu().numpy(), wt.cpu().numpy(), idx_ref, w_ref, gap, z_ref, b, w.n_group,
                             w.topk_group, w.top_k)
    rows = [r for r in P.sample_tokens(idx_ref, n_extra=4, seed=w.T) if same[r]][:48]
    y_ref = oracle.moe_rows(x[rows], idx_ref[rows], w_ref[rows], _experts_host(w, np.unique(idx_ref[rows])), w.E)
    ref = oracle.post_residual(y_ref, pw, eps, resid[rows], layer)
    _, add = _factors(layer)
    rms_all = np.sqrt(np.mean(y_ref ** 2))
    rms_row = np.sqrt(np.mean(y_ref ** 2, axis=1, keepdims=True))
    wmax = np.max(np.abs(synth_bf16(pw)))
    # n = y * w / rms_row(y): an error of at most dy = Y_TOL * rms_all in y moves y / rms_row by
    # dy / rms_row directly and by at most max|y_row| / rms_row * dy / rms_row through the
    # row's rms; times the weight and the residual factor 1/sqrt(k)
    amax = np.max(np.abs(y_ref), axis=1, keepdims=True)
    tol = add * wmax * (P.Y_TOL * rms_all / rms_row) * (1 + amax / rms_row) * 1.05
    err = np.abs(got[rows] - ref)
    print("%s: %d sampled rows, max err %.3e, min tol %.3e" % (name, len(rows), err.max(), tol.min()))
    assert (err <= tol).all()


def synth_bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
