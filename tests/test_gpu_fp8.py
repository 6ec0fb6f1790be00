"""FP8 (OCP E4M3 + per-32 E8M0 scales) expert weights on the GPU, through the C ABI.

The quantizer is integer/byte work: bit-exact against the oracle's. The layer with FP8
weights is the bf16 layer on the dequantized weights: the oracle quantizes the host
weights itself, dequantizes them and runs its usual layer, and the GPU output must agree
within the layer's y bar."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from synth.recipes import Workload
from tests import _parity as P
from tests.test_gpu_parity import _shape, _oracle_inputs, _random_workload

pytestmark = pytest.mark.gpu

MID = Workload(30, "mid_fp8_T77", T=77, d=512, E=256, n_group=8, topk_group=4, top_k=8, I=512)


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _quantize_dev(w_dev, rows, K):
    q = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    moe.beam_moe_quantize_fp8(rows, K, w_dev, q, s)
    return q, s


def test_quantize_bitexact():
    """Random expert rows plus edge blocks: zeros, tiny values, values past the largest code."""
    print("case quantize", flush=True)
    w = MID
    wg, _, wd = synth.expert_weights(w, 3)
    edge = np.zeros((4, w.d), dtype=np.uint16)
    edge[1, :32] = 0x0001                      # bf16 subnormals
    edge[1, 32:64] = 0x8080                    # -2^-126
    vals = np.linspace(-3.0, 3.0, w.d - 64).astype(np.float32)
    edge[2, 64:] = (vals.view(np.uint32) >> 16).astype(np.uint16)
    edge[3, :] = 0x3F80                        # all 1.0
    edge[3, 5] = 0x43E8                        # 464: block max in the saturating range
    for name, mat in (("Wg", wg), ("Wd", wd), ("edge", edge)):
        rows, K = mat.shape
        q, s = _quantize_dev(_bits_dev(mat), rows, K)
        torch.cuda.synchronize()
        q_ref, s_ref = oracle.fp8_quantize(mat)
        assert np.array_equal(s.cpu().numpy(), s_ref), name
        assert np.array_equal(q.cpu().numpy(), q_ref), name


def _gpu_fp8_forward(w, t):
    shape = _shape(w)
    rows_gu, rows_d = w.E * w.I, w.E * w.d
    qg, sg = _quantize_dev(t["Wg"], rows_gu, w.d)
    qu, su = _quantize_dev(t["Wu"], rows_gu, w.d)
    qd, sd = _quantize_dev(t["Wd"], rows_d, w.I)
    ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    y = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    hid = t["h"] if w.prenorm else t["x"]
    moe.beam_moe_forward_fp8(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], qg, qu, qd, sg, su, sd, y, idx, wt,
                             None, ws)
    y0 = torch.empty_like(y)
    moe.beam_moe_forward(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], t["Wg"], t["Wu"], t["Wd"], y0, None, None,
                         None, ws)
    # packed codes (two codes per 16-bit unit through beam_moe_pack_weights): bitwise the same layer
    packed = []
    for q, rows, K in ((qg, rows_gu, w.d), (qu, rows_gu, w.d), (qd, rows_d, w.I)):
        p = torch.empty_like(q)
        moe.beam_moe_pack_weights(rows, K // 2, q, p)
        packed.append(p)
    shape_pk = moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob, w.eps,
                              weight_layout=moe.WEIGHTS_PACKED)
    y_pk = torch.full_like(y, float("nan"))
    moe.beam_moe_forward_fp8(shape_pk, hid, t.get("norm_w"), t["Wr"], t["bias"], *packed, sg, su, sd, y_pk, None,
                             None, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_pk), "packed fp8 codes changed the layer output"
    return y.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy(), y0.cpu().numpy()


def _fp8_experts(w, ids):
    out = {}
    for e in ids:
        wg, wu, wd = synth.expert_weights(w, int(e))
        out[int(e)] = tuple(oracle.fp8_dequantize(*oracle.fp8_quantize(m)) for m in (wg, wu, wd))
    return out


def _random_fp8_workload(i):
    """A seeded random supported shape, with d and I multiples of 512 (the FP8 kernels' k steps)
    and few enough tokens per expert for the weight streams."""
    from dataclasses import replace
    rng = np.random.default_rng(777 + i)
    w = _random_workload(i)
    T = min(w.T, max(1, 16 * w.E // w.top_k))
    return replace(w, cfg_id=80 + i, name="random_fp8_%d" % i, T=T, d=int(rng.choice([512, 1024])),
                   I=int(rng.choice([512, 1024])))


@pytest.mark.parametrize("cfg", ["mid", 1] + ["random_%d" % i for i in range(4)])
def test_forward_fp8_parity(cfg):
    if isinstance(cfg, str) and cfg.startswith("random_"):
        w = _random_fp8_workload(int(cfg.split("_")[1]))
    else:
        w = MID if cfg == "mid" else recipes.WORKLOADS[cfg]
    print("case forward_fp8", w.name, w, flush=True)
    t = synth.device_inputs(w)
    y, idx, wt, y_bf16 = _gpu_fp8_forward(w, t)
    del t
    x, Wr, b = _oracle_inputs(w)
    idx_ref, w_ref, gap, z_ref = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale,
                                              w.norm_topk_prob, want_logits=True)
    same = P.compare_routing(idx, wt, idx_ref, w_ref, gap, z_ref, b, w.n_group, w.topk_group, w.top_k)
    # every token at the mid shape; at the Beam shape a sample (each token's 8 experts are
    # generated, quantized and run on the host)
    rows = np.arange(w.T) if w.d <= 1024 else P.sample_tokens(idx_ref, n_extra=6, seed=7)
    rows = np.array([r for r in rows if same[r]])
    experts = _fp8_experts(w, np.unique(idx_ref[rows]))
    y_ref = oracle.moe_rows(x[rows], idx_ref[rows], w_ref[rows], experts, w.E)
    err, rms = P.output_error(y[rows], y_ref)
    qerr = np.sqrt(np.mean((y - y_bf16) ** 2)) / np.sqrt(np.mean(y_bf16 ** 2))
    print("%s fp8: %d tokens, max|dy| %.3e, rms %.3e; fp8 vs bf16 weights: rel rms %.3e"
          % (w.name, len(rows), err, rms, qerr))
    assert np.isfinite(y).all()
    assert err <= P.Y_TOL * rms
