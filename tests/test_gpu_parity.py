"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Small and mid-sized shapes are compared on every token; the Beam-shape workloads
(T = 64, 8192, 4096 skewed, 32768 with the fused pre-norm) are compared on every
token for routing and on a deterministic sample of tokens for the layer output,
plus properties that hold at any size (determinism, full overwrite)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from synth.recipes import Workload
from tests import _parity as P

pytestmark = pytest.mark.gpu

_MID = dict(d=512, E=256, n_group=8, topk_group=4, top_k=8, I=256)
SMALL = {
    "tiny": recipes.WORKLOADS[0],
    "mid_T1": Workload(20, "mid_T1", T=1, **_MID),
    "mid_T77": Workload(21, "mid_T77", T=77, **_MID),
    "mid_T2000": Workload(22, "mid_T2000", T=2000, **_MID),
    "mid_skew_T600": Workload(23, "mid_skew_T600", T=600, hot_experts=16, hot_bias=0.5, **_MID),
    "mid_prenorm_T333": Workload(24, "mid_prenorm_T333", T=333, prenorm=True, **_MID),
    "e128_T300": Workload(25, "e128_T300", T=300, d=256, E=128, n_group=4, topk_group=2, top_k=6, I=128),
    "e1024_T200": Workload(26, "e1024_T200", T=200, d=256, E=1024, n_group=16, topk_group=4, top_k=16, I=64),
    "e64_T150": Workload(27, "e64_T150", T=150, d=128, E=64, n_group=8, topk_group=3, top_k=5, I=64),
    "mid_nonorm_T100": Workload(28, "mid_nonorm_T100", T=100, norm_topk_prob=False, **_MID),
    # concentrated routing: 8 experts with a +5 bias take most pairs, so single experts see every
    # token (the weight streams' multi-tile loop; the GEMM's many m-tiles of one expert)
    "mid_conc_T64": Workload(29, "mid_conc_T64", T=64, hot_experts=8, hot_bias=5.0, **_MID),
    "mid_conc_T2000": Workload(30, "mid_conc_T2000", T=2000, hot_experts=8, hot_bias=5.0, **_MID),
    # degenerate routing shapes: every group kept (plain top-k), one expert per token, no groups
    "e64_allgroups_T100": Workload(31, "e64_allgroups_T100", T=100, d=128, E=64, n_group=8, topk_group=8, top_k=6,
                                   I=64),
    "k1_T100": Workload(32, "k1_T100", T=100, d=256, E=32, n_group=4, topk_group=2, top_k=1, I=128),
    "g1_T100": Workload(33, "g1_T100", T=100, d=256, E=256, n_group=1, topk_group=1, top_k=8, I=128),
    # d not a multiple of 128: many tokens per expert but no tiled GEMM, so the weight streams
    # run 16-token tile after tile
    "d192_T500": Workload(34, "d192_T500", T=500, d=192, E=16, n_group=4, topk_group=2, top_k=4, I=192),
    # from T = 2048 the router product runs on the tiled GEMM, k cut into parts: d = 512 gives
    # eight one-stage parts; E = 128 leaves the second 256-row block of its 384 weight rows
    # half past the end
    "mid_T2100": Workload(35, "mid_T2100", T=2100, **_MID),
    "e128_T2100": Workload(36, "e128_T2100", T=2100, d=256, E=128, n_group=4, topk_group=2, top_k=6, I=128),
    # d = 2048 below T = 1024: 16 k parts per logit, so the top-k adds them a quarter per wave, and
    # 16 token blocks x 16 parts still take the router path that splits the FP32 weight in registers
    "d2048_T1000": Workload(37, "d2048_T1000", T=1000, d=2048, E=256, n_group=8, topk_group=4, top_k=8, I=128),
    # d = 2304 at T = 64: k in 18 parts, so the quarter-split top-k adds uneven quarters (5, 5, 5, 3)
    # and the in-register router weight split runs at 18 parts
    "d2304_T64": Workload(38, "d2304_T64", T=64, d=2304, E=256, n_group=8, topk_group=4, top_k=8, I=128),
}
BEAM = {i: recipes.WORKLOADS[i] for i in (1, 2, 3, 4)}


def _shape(w):
    return moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob, w.eps)


def _eps32(w):
    """The eps the kernels see (the ABI carries it as FP32)."""
    return float(np.float32(w.eps))


def _gpu_forward(w, t, shape=None):
    shape = shape or _shape(w)
    dev = t["Wr"].device
    ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    y = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((w.T, w.top_k), -7, dtype=torch.int32, device=dev)
    wt = torch.full((w.T, w.top_k), float("nan"), dtype=torch.float32, device=dev)
    z = torch.full((w.T, w.E), float("nan"), dtype=torch.float32, device=dev)
    hid = t["h"] if w.prenorm else t["x"]
    moe.beam_moe_forward(shape, hid, t.get("norm_w"), t["Wr"], t["bias"], t["Wg"], t["Wu"], t["Wd"], y, idx, wt, z, ws)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), idx=idx.cpu().numpy(), w=wt.cpu().numpy(), z=z.cpu().numpy())


def _oracle_inputs(w):
    x = synth.hidden(w)
    if w.prenorm:
        x = oracle.rmsnorm(x, synth.norm_weight(w), _eps32(w))
    return x, synth.router_weight(w), synth.bias(w)


def _experts_host(w, ids):
    return {int(e): synth.expert_weights(w, int(e)) for e in ids}


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------------------

def test_synth_device_matches_host():
    """The two twins of the input generator agree bit for bit on every tensor kind."""
    dev = torch.device("cuda")
    w = recipes.WORKLOADS[2]
    for tid, std, dtype, start, n in [(recipes.TID_X, 1.0, synth.BF16, 0, 1 << 20),
                                     (recipes.TID_WG, w.std_in, synth.BF16, 255 * w.I * w.d + 12345, 1 << 20),
                                     (recipes.TID_WD, w.std_down, synth.BF16, 77 * w.I * w.d, 1 << 20),
                                     (recipes.TID_WR, w.std_in, synth.F32, 0, w.d * w.E)]:
        buf = torch.empty(n, dtype=torch.float32 if dtype == synth.F32 else torch.int16, device=dev)
        synth.dev_normal(buf.data_ptr(), n, w.seed, tid, 0.0, std, dtype, start=start,
                         stream=torch.cuda.current_stream().cuda_stream)
        got = buf.cpu().numpy().view(np.float32 if dtype == synth.F32 else np.uint16)
        ref = synth.host_normal(n, w.seed, tid, 0.0, std, dtype, start=start)
        assert np.array_equal(got, ref), "tensor id %d differs" % tid
    buf = torch.empty(4096, dtype=torch.float32, device=dev)
    synth.dev_uniform(buf.data_ptr(), 4096, 7, recipes.TID_BIAS, -0.1, 0.1, synth.F32,
                      stream=torch.cuda.current_stream().cuda_stream)
    assert np.array_equal(buf.cpu().numpy(), synth.host_uniform(4096, 7, recipes.TID_BIAS, -0.1, 0.1, synth.F32))


def _random_workload(i):
    """A seeded random shape from the whole supported range (include/beam_moe.h): E up to 64
    with power-of-two group sizes, or E in {128, 256, 512} with power-of-two group counts; any
    topk_group and top_k they allow; d, I multiples of 64; ragged T (past 2048 the router runs on
    the tiled GEMM); random scale, normalisation, pre-norm and hot experts."""
    rng = np.random.default_rng(4242 + i)
    E = int(rng.choice([8, 16, 24, 32, 48, 64, 128, 256, 512]))
    if E <= 64:
        gsz = int(rng.choice([g for g in (2, 4, 8, 16, 32, 64) if E % g == 0]))
        G = E // gsz
    else:
        G = int(rng.choice([g for g in (1, 2, 4, 8, 16, 32, 64) if E // g >= 2]))
    KG = int(rng.integers(1, G + 1))
    K = int(rng.integers(1, min(16, KG * (E // G)) + 1))
    d = int(rng.choice([64, 128, 192, 256, 384, 512]))
    I = int(rng.choice([64, 128, 192, 256]))
    T = int(rng.choice([1, 2, 7, 16, 33, 64, 65, 100, 255, 256, 257, 511, 700, 1200, 2100]))
    while T * K > 12000:
        T //= 2
    hot = int(rng.integers(0, E // 4 + 1)) if rng.random() < 0.3 else 0
    return Workload(60 + i, "random_%d" % i, T=T, d=d, E=E, n_group=G, topk_group=KG, top_k=K, I=I,
                    scale=float(rng.uniform(0.5, 3.0)), norm_topk_prob=bool(rng.random() < 0.7),
                    hot_experts=hot, hot_bias=0.3 if hot else 0.0, prenorm=bool(rng.random() < 0.3))


def _check_every_token(w, name):
    print("case", name, w, flush=True)
    t = synth.device_inputs(w)
    g = _gpu_forward(w, t)
    x, Wr, b = _oracle_inputs(w)
    idx_ref, w_ref, gap, z_ref = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale,
                                              w.norm_topk_prob, want_logits=True)
    np.testing.assert_allclose(g["z"], z_ref, rtol=0, atol=1e-4)
    same = P.compare_routing(g["idx"], g["w"], idx_ref, w_ref, gap, z_ref, b, w.n_group, w.topk_group, w.top_k)
    experts = _experts_host(w, np.unique(idx_ref))
    rows = np.nonzero(same)[0]
    y_ref = oracle.moe_rows(x[rows], idx_ref[rows], w_ref[rows], experts, w.E)
    err, rms = P.output_error(g["y"][rows], y_ref)
    print("%s: excused %d, max|dy| %.3e, rms %.3e" % (name, (~same).sum(), err, rms))
    assert np.isfinite(g["y"]).all()
    assert err <= P.Y_TOL * rms


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity_small(name):
    """Whole layer on every token: routing, weights, logits and y against the oracle."""
    _check_every_token(SMALL[name], name)


@pytest.mark.parametrize("i", range(16))
def test_forward_parity_random_shape(i):
    """Whole layer on every token at a seeded random supported shape."""
    _check_every_token(_random_workload(i), "random_%d" % i)


# rows per compared block of each expert's segment, each expert's last row compared too: every
# m-tile of the tiled GEMMs holds a compared token, as a full tile (256 or 320 rows from the
# expert's first row) spans a whole block and the expert's last tile holds its last row
_COVER_BLOCK = {2: 64, 3: 64, 4: 128}


def _host_bf16(a):
    return a.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_rows_by_share(w, t, x_rows, idx_rows, w_rows, span=32):
    """Oracle y for the given rows, summed over expert-parallel shares of `span` experts, so only one
    share's expert weights sit in host memory at a time (the shares of a partition add up to the
    whole layer: a pinned property of the oracle). The weights come from the device tensors the
    seeded generator filled (its device twin is pinned bit for bit against the host twin)."""
    y = np.zeros((len(x_rows), w.d))
    used = set(np.unique(idx_rows).tolist())
    for e0 in range(0, w.E, span):
        ids = [e for e in range(e0, min(w.E, e0 + span)) if e in used]
        if not ids:
            continue
        experts = {e: (_host_bf16(t["Wg"][e]), _host_bf16(t["Wu"][e]), _host_bf16(t["Wd"][e])) for e in ids}
        y += oracle.moe_share_rows(x_rows, idx_rows, w_rows, experts, e0, min(span, w.E - e0))
    return y


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_forward_parity_beam(cfg):
    """Beam shape: routing on every token; y on every token at T=64, and at the prefill sizes on a
    set of tokens that puts a compared row in every block of 64 (T=8192, T=4096 skewed) or 128
    (T=32768) rows of every expert's segment, each expert's last row included, so every work
    item of the grouped GEMMs (each m-tile of each expert, through all n-blocks) is checked;
    run-to-run determinism."""
    w = BEAM[cfg]
    print("case beam cfg", cfg, "T", w.T, flush=True)
    t = synth.device_inputs(w)
    g = _gpu_forward(w, t)
    x, Wr, b = _oracle_inputs(w)
    idx_ref, w_ref, gap, z_ref = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale,
                                              w.norm_topk_prob, want_logits=True)
    np.testing.assert_allclose(g["z"], z_ref, rtol=0, atol=1e-4)
    same = P.compare_routing(g["idx"], g["w"], idx_ref, w_ref, gap, z_ref, b, w.n_group, w.topk_group, w.top_k)
    if cfg in _COVER_BLOCK:
        # the GPU's own routing decides the GEMM tiles; cover them (excused tokens are left out below)
        cover = P.cover_tokens(g["idx"], w.E, _COVER_BLOCK[cfg])
    else:
        cover = np.arange(w.T)
    rows = np.array([r for r in cover if same[r]], dtype=np.int64)
    y_ref = _oracle_rows_by_share(w, t, x[rows], idx_ref[rows], w_ref[rows])
    err, rms = P.output_error(g["y"][rows], y_ref)
    print("cfg %d: excused %d of %d, compared %d tokens (cover %d), max|dy| %.3e, rms %.3e, ratio %.2e"
          % (cfg, (~same).sum(), w.T, len(rows), len(cover), err, rms, err / rms))
    assert len(rows) >= len(cover) - 4
    assert err <= P.Y_TOL * rms
    assert np.isfinite(g["y"]).all()
    g2 = _gpu_forward(w, t)
    assert np.array_equal(g2["y"].view(np.uint32), g["y"].view(np.uint32)), "run-to-run output differs"
    assert np.array_equal(g2["idx"], g["idx"])


def test_route_prenorm_x_bitwise():
    """The fused pre-MLP RMSNorm (FP64 on the GPU) gives the oracle's bf16 x bit for bit."""
    w = BEAM[4].with_T(2048)
    t = synth.device_inputs(w)
    shape = _shape(w)
    dev = t["Wr"].device
    ws = torch.empty(moe.beam_moe_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    xn = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((w.T, w.top_k), dtype=torch.int32, device=dev)
    wt = torch.empty((w.T, w.top_k), dtype=torch.float32, device=dev)
    moe.beam_moe_route(shape, t["h"], t["norm_w"], xn, t["Wr"], t["bias"], idx, wt, None, ws)
    torch.cuda.synchronize()
    got = xn.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.rmsnorm(synth.hidden(w), synth.norm_weight(w), _eps32(w))
    assert np.count_nonzero(got != ref) == 0


def _dispatch_gpu(idx_np, E, T, K):
    w = Workload(99, "dispatch", T=T, d=64, E=E, n_group=max(1, E // 4) if E // 4 <= 64 else 16,
                 topk_group=1, top_k=K, I=64)
    shape = moe.make_shape(T, 64, E, w.n_group, w.n_group, K, 64)
    dev = torch.device("cuda")
    ws = torch.empty(max(moe.beam_moe_workspace_bytes(shape), 256), dtype=torch.uint8, device=dev)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).to(dev)
    off = torch.full((E + 1,), -5, dtype=torch.int32, device=dev)
    sp = torch.full((T * K,), -5, dtype=torch.int32, device=dev)
    pr = torch.full((T * K,), -5, dtype=torch.int32, device=dev)
    moe.beam_moe_dispatch(shape, idx, off, sp, pr, ws)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy(), pr.cpu().numpy()


@pytest.mark.parametrize("T,K,E,law", [
    (1, 8, 256, "uniform"), (64, 8, 256, "uniform"), (128, 8, 256, "uniform"), (129, 8, 256, "uniform"),
    (1000, 8, 256, "uniform"), (8192, 8, 256, "skew"), (4099, 4, 16, "uniform"), (333, 16, 1024, "uniform"),
    (5000, 8, 256, "one_hot_expert"),
])
def test_dispatch_parity(T, K, E, law):
    """Counting sort vs a stable sort, on seeded expert ids (small and chunked paths)."""
    rng = np.random.default_rng(T * 31 + K)
    if law == "uniform":
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    elif law == "skew":
        p = rng.dirichlet(np.full(E, 0.3))
        idx = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)])
    else:  # every token lists expert 7 first: one segment of T pairs
        idx = np.stack([np.concatenate([[7], rng.choice(np.setdiff1d(np.arange(E), [7]), K - 1, replace=False)])
                        for _ in range(T)])
    off, sp, pr = _dispatch_gpu(idx, E, T, K)
    o_ref, sp_ref, pr_ref = oracle.dispatch(idx, E)
    assert np.array_equal(off, o_ref)
    assert np.array_equal(sp, sp_ref)
    assert np.array_equal(pr, pr_ref)


def test_dispatch_drops_out_of_range_ids():
    T, K, E = 300, 4, 16
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[3, 1] = -1
    idx[200, 0] = E
    idx[299, 3] = 1 << 20
    off, sp, pr = _dispatch_gpu(idx, E, T, K)
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    assert off[E] == valid.sum()
    assert np.array_equal(sp[:off[E]], order)
    assert np.all(sp[off[E]:] == -1)
    assert np.all(pr[~valid] == -1)
    assert np.array_equal(pr[order], np.arange(valid.sum()))


def test_identical_experts_beam_decode():
    """All 256 experts equal: y = 2.5 * expert(x) for every token, whatever the routing."""
    w = BEAM[1]
    t = synth.device_inputs(w)
    for k in ("Wg", "Wu", "Wd"):
        t[k][1:] = t[k][0:1]
    g = _gpu_forward(w, t)
    wg, wu, wd = synth.expert_weights(w, 0)
    x, _, _ = _oracle_inputs(w)
    o = oracle.expert(x, wg, wu, wd)
    err, rms = P.output_error(g["y"], w.scale * o)
    print("identical experts: max|dy| %.3e rms %.3e" % (err, rms))
    assert err <= P.Y_TOL * rms


@pytest.mark.parametrize("name", ["mid_T77", "mid_T2000"])
def test_doubled_down_projection_doubles_y(name):
    """Wd -> 2 Wd (exact in bf16) doubles y bit for bit: the routing does not see Wd, and every
    product and sum after it scales by a power of two. T=77 runs the weight streams, T=2000 the
    tiled GEMM; both on row-major and on packed weights."""
    w = SMALL[name]
    print("case doubled Wd", name, flush=True)
    t = synth.device_inputs(w)
    g = _gpu_forward(w, t)
    t2 = dict(t)
    t2["Wd"] = t["Wd"] * 2
    g2 = _gpu_forward(w, t2)
    assert np.array_equal(g2["idx"], g["idx"])
    assert np.isfinite(g["y"]).all()
    assert np.array_equal(g2["y"].view(np.uint32), (2 * g["y"]).view(np.uint32))
    shape = moe.make_shape(w.T, w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I, w.scale, w.norm_topk_prob, w.eps,
                           weight_layout=moe.WEIGHTS_PACKED)
    t3 = dict(t2)
    t3["Wg"], t3["Wu"], t3["Wd"] = moe.pack_expert_weights(t["Wg"], t["Wu"], t2["Wd"])
    g3 = _gpu_forward(w, t3, shape)
    assert np.array_equal(g3["y"].view(np.uint32), g2["y"].view(np.uint32))


def test_token_permutation_equivariance():
    """Permuting tokens permutes y bit for bit (no cross-token arithmetic)."""
    w = SMALL["mid_T2000"]
    t = synth.device_inputs(w)
    g = _gpu_forward(w, t)
    perm = np.random.default_rng(0).permutation(w.T)
    t2 = dict(t)
    t2["x"] = t["x"][torch.from_numpy(perm).to(t["x"].device)].contiguous()
    g2 = _gpu_forward(w, t2)
    assert np.array_equal(g2["idx"], g["idx"][perm])
    assert np.array_equal(g2["y"].view(np.uint32), g["y"][perm].view(np.uint32))


def test_zero_tokens_is_noop():
    w = SMALL["mid_T77"].with_T(0)
    shape = _shape(w)
    assert moe.beam_moe_forward(shape, 16, None, 16, 16, 16, 16, 16, 16, None, None, None, None) == 0
