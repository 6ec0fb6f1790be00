"""Packed expert weights (beam_moe_pack_weights, weight_layout = BEAM_MOE_WEIGHTS_PACKED) on
the GPU, through the C ABI. The packing is checked bit for bit against the layout the header
defines (rebuilt here with numpy); every entry point that takes the packed layout must give
results bitwise equal to the row-major call on the same values (the kernels feed the same
operands to the same MFMAs in the same order), and one mid-size layer is checked against
the oracle directly."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from tests import _parity as P
from tests.test_gpu_parity import SMALL, _oracle_inputs, _experts_host

pytestmark = pytest.mark.gpu


def _pack_reference(w):
    """The header's packed layout, from its definition: block b, step j, lane l holds
    w[16b + l % 16, 32j + 8(l // 16) : +8]."""
    rows, K = w.shape
    out = np.empty(rows * K, dtype=w.dtype)
    o = 0
    for b in range(rows // 16):
        for j in range(K // 32):
            for l in range(64):
                out[o:o + 8] = w[16 * b + l % 16, 32 * j + 8 * (l // 16): 32 * j + 8 * (l // 16) + 8]
                o += 8
    return out


def _shape(w, layout):
    return moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob, w.eps,
                          weight_layout=layout)


def _forward(w, t, layout, W):
    shape = _shape(w, layout)
    ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    y = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((w.T, w.top_k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((w.T, w.top_k), float("nan"), dtype=torch.float32, device="cuda")
    hid = t["h"] if w.prenorm else t["x"]
    moe.beam_moe_forward(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], *W, y, idx, wt, None, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rows,K", [(16, 32), (48, 96), (64, 5120), (2560, 64)])
def test_pack_layout_bit_exact(rows, K):
    rng = np.random.default_rng(rows + K)
    w = rng.integers(0, 1 << 16, size=(rows, K), dtype=np.uint16)
    wd = torch.from_numpy(w.view(np.int16)).cuda()
    pd = torch.full((rows * K,), -1, dtype=torch.int16, device="cuda")
    moe.beam_moe_pack_weights(rows, K, wd, pd)
    torch.cuda.synchronize()
    assert np.array_equal(pd.cpu().numpy().view(np.uint16), _pack_reference(w))


def test_pack_beam_expert_slab():
    """Two experts of the Beam gate projection: blocks and steps at the real sizes."""
    w = recipes.WORKLOADS[1]
    t = synth.device_inputs(w)
    slab = t["Wg"][5:7].contiguous()
    p = torch.empty_like(slab)
    moe.beam_moe_pack_weights(2 * w.I, w.d, slab, p)
    torch.cuda.synchronize()
    host = slab.view(torch.int16).cpu().numpy().view(np.uint16).reshape(2 * w.I, w.d)
    got = p.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    rows = [0, 15, 16, 2559, 2560, 5119]
    for r in rows:
        b, rr = divmod(r, 16)
        for j in (0, 1, 77, w.d // 32 - 1):
            for c in range(4):
                l = rr + 16 * c
                o = ((b * (w.d // 32) + j) * 64 + l) * 8
                assert np.array_equal(got[o:o + 8], host[r, 32 * j + 8 * c: 32 * j + 8 * c + 8])


@pytest.mark.parametrize("name", ["tiny", "mid_T77", "mid_T2000", "mid_prenorm_T333", "e128_T300", "e64_T150",
                                  "e1024_T200", "mid_conc_T64", "mid_conc_T2000"])
def test_forward_packed_bitwise_small(name):
    w = SMALL[name]
    print("case packed", name, flush=True)
    t = synth.device_inputs(w)
    rm = _forward(w, t, moe.WEIGHTS_ROW_MAJOR, (t["Wg"], t["Wu"], t["Wd"]))
    pk = _forward(w, t, moe.WEIGHTS_PACKED, moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]))
    for a, b in zip(rm, pk):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_forward_packed_against_oracle_mid():
    w = SMALL["mid_T77"]
    t = synth.device_inputs(w)
    y, idx, wt = _forward(w, t, moe.WEIGHTS_PACKED, moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]))
    x, Wr, b = _oracle_inputs(w)
    idx_ref, w_ref, gap, z_ref = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale,
                                              w.norm_topk_prob, want_logits=True)
    assert np.array_equal(idx, idx_ref)
    ref = oracle.moe_rows(x, idx_ref, w_ref, _experts_host(w, range(w.E)), w.E)
    err, rms = P.output_error(y, ref)
    assert err <= P.Y_TOL * rms


# d = I = 512: both grouped GEMMs take the weight-streaming form on packed weights (k runs of 512)
# and the LDS-staged form on row-major ones; four hot experts get several 256-token m-tiles each,
# the last ragged, and the cold ones partial tiles of every live-subtile count
# d = 384, I = 512: the down pass streams weights (k = I) over n-blocks of 256 output channels, the
# second of which runs past d (its waves read a clamped block and store nothing); gate/up (k = d)
# stays on the LDS-staged GEMM
# ws_mid_T1500: both expert GEMMs on the weight-streaming kernel, tiles of 320 tokens whose live
# 16-token subtile counts (oracle routing) take every value 2, 4, .., 20; ws_d384_T800: gate/up on
# the LDS-staged kernel (d not a multiple of 512), down weight-streaming on tiles of 256.
# The weight-streaming launches are persistent (one block per CU walks its XCD's range of items):
# ws_e2_T40 has fewer items than XCDs (gate/up 8, down 4: XCD ranges of one item or none);
# ws_mid_T4000 gives each block several items of different tile heights, and the blocks whose
# XCD range runs out first take items from the other ranges.
WS_CASES = {
    "ws_e2_T40": recipes.Workload(44, "ws_e2_T40", T=40, d=512, E=2, n_group=1, topk_group=1, top_k=1, I=512),
    "ws_mid_T4000": recipes.Workload(45, "ws_mid_T4000", T=4000, d=512, E=64, n_group=8, topk_group=4, top_k=8,
                                     I=512),
    "ws_mid_T1500": recipes.Workload(42, "ws_mid_T1500", T=1500, d=512, E=64, n_group=8, topk_group=4, top_k=8,
                                     I=512, hot_experts=4, hot_bias=0.5),
    "ws_d384_T800": recipes.Workload(43, "ws_d384_T800", T=800, d=384, E=32, n_group=4, topk_group=2, top_k=4,
                                     I=512),
}


@pytest.mark.parametrize("name", sorted(WS_CASES))
def test_weight_streaming_gemms_every_token(name):
    """The weight-streaming grouped GEMMs against the oracle on every token, and bitwise equal to
    the LDS-staged GEMMs on the same values in the row-major layout."""
    w = WS_CASES[name]
    assert w.T * w.top_k > 16 * w.E                     # the tiled GEMM path
    print("case packed", w.name, flush=True)
    t = synth.device_inputs(w)
    rm = _forward(w, t, moe.WEIGHTS_ROW_MAJOR, (t["Wg"], t["Wu"], t["Wd"]))
    pk = _forward(w, t, moe.WEIGHTS_PACKED, moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"]))
    for a, b in zip(rm, pk):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    y, idx, wt = pk
    counts = np.bincount(idx.reshape(-1), minlength=w.E)
    if w.hot_experts:
        assert counts.max() > 2 * 256 and (counts[counts > 0] % 256).min() < 32   # several m-tiles; small tails
    x, Wr, b = _oracle_inputs(w)
    idx_ref, w_ref, gap, z_ref = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale,
                                              w.norm_topk_prob, want_logits=True)
    same = P.compare_routing(idx, wt, idx_ref, w_ref, gap, z_ref, b, w.n_group, w.topk_group, w.top_k)
    rows = np.nonzero(same)[0]
    ref = oracle.moe_rows(x[rows], idx_ref[rows], w_ref[rows], _experts_host(w, range(w.E)), w.E)
    err, rms = P.output_error(y[rows], ref)
    print("%s: compared %d of %d tokens, max|dy| %.3e, rms %.3e" % (w.name, len(rows), w.T, err, rms))
    assert len(rows) >= w.T - 4
    assert err <= P.Y_TOL * rms


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_forward_packed_bitwise_beam(cfg):
    """Every Beam workload (decode streams; prefill, skewed and large-chunk grouped GEMMs): packed
    equals row-major bit for bit."""
    w = recipes.WORKLOADS[cfg]
    print("case packed beam", w.name, flush=True)
    t = synth.device_inputs(w)
    rm = _forward(w, t, moe.WEIGHTS_ROW_MAJOR, (t["Wg"], t["Wu"], t["Wd"]))
    W = moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"])
    for k in ("Wg", "Wu", "Wd"):          # only the packed copies stay resident
        del t[k]
    torch.cuda.empty_cache()
    pk = _forward(w, t, moe.WEIGHTS_PACKED, W)
    for a, b in zip(rm, pk):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_residual_and_share_packed_bitwise():
    """The fused post-norm + residual layer and an expert-parallel share read packed weights too."""
    w = recipes.WORKLOADS[1]
    t = synth.device_inputs(w)
    Wp = moe.pack_expert_weights(t["Wg"], t["Wu"], t["Wd"])
    resid = torch.from_numpy(synth.residual(w)).cuda()
    pw = torch.from_numpy(synth.post_norm_weight(w).view(np.int16)).cuda().view(torch.bfloat16)
    outs = []
    for layout, W in ((moe.WEIGHTS_ROW_MAJOR, (t["Wg"], t["Wu"], t["Wd"])), (moe.WEIGHTS_PACKED, Wp)):
        shape = _shape(w, layout)
        ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        out = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
        idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
        wt = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
        moe.beam_moe_forward_residual(shape, t["x"], None, t["Wr"], t["bias"], *W, pw, 7, resid, out, None, idx, wt,
                                      None, ws)
        e0, n = 96, 32
        sws = torch.empty(moe.beam_moe_share_workspace_bytes(shape, n), dtype=torch.uint8, device="cuda")
        yp = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
        moe.beam_moe_experts_share(shape, e0, n, t["x"], idx, wt, W[0][e0:e0 + n], W[1][e0:e0 + n],
                                   W[2][e0:e0 + n], yp, sws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), yp.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
