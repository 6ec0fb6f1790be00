"""Expert-parallel share on the GPU (beam_moe_experts_share, through the C ABI) against the
oracle's moe_share_rows (double) on the GPU's own routing ("Use HF Transformers" cookbook,
Parallelism: each GPU holds one block of the experts). Every token at small sizes, for the
routing groups and for unaligned, one-expert and empty blocks; at the Beam shapes a token
sample per block, and on every token the partition property: the shares of the 8 groups add
up to beam_moe_forward's y (the same kernels, the slot sum split in a different order)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import sparse_moe_layer_beam_amd as moe
from synth import recipes
from tests import _parity as P
from tests.test_gpu_parity import SMALL, _gpu_forward, _oracle_inputs, _experts_host, _shape, _random_workload

pytestmark = pytest.mark.gpu

# FP32 re-association of at most top_k terms per element (the shares' slot sums are added
# per block, the layer's in slot order), relative to the largest |y| of the run
PARTITION_TOL = 1e-5


def _share(w, t, shape, e0, n, idx_d, w_d):
    ws = torch.empty(max(1, moe.beam_moe_share_workspace_bytes(shape, n)), dtype=torch.uint8, device="cuda")
    y = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.beam_moe_experts_share(shape, e0, n, t["x"], idx_d, w_d, t["Wg"][e0:e0 + n], t["Wu"][e0:e0 + n],
                               t["Wd"][e0:e0 + n], y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check_block(y_gpu, ref, label):
    assert np.isfinite(y_gpu).all(), label
    err, rms = P.output_error(y_gpu, ref)
    print("%s: max|dy| %.3e, rms %.3e" % (label, err, rms))
    if rms == 0.0:
        assert np.all(y_gpu == 0.0), label
    else:
        assert err <= P.Y_TOL * rms, label


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["tiny", "mid_T77", "mid_T2000", "e64_T150"] + ["random_%d" % i for i in range(4)])
def test_share_small_every_token(name):
    if name.startswith("random_"):      # the share takes the layer's input x as it is: no pre-norm
        from dataclasses import replace
        w = replace(_random_workload(int(name.split("_")[1])), prenorm=False)
    else:
        w = SMALL[name]
    print("case share", name, w, flush=True)
    t = synth.device_inputs(w)
    shape = _shape(w)
    full = _gpu_forward(w, t, shape)
    idx_d = torch.from_numpy(full["idx"]).cuda()
    w_d = torch.from_numpy(full["w"]).cuda()
    x = synth.hidden(w)
    experts = _experts_host(w, range(w.E))
    gs = w.E // w.n_group
    blocks = [(g * gs, gs) for g in range(w.n_group)]
    tot = np.zeros((w.T, w.d))
    for e0, n in blocks:
        y = _share(w, t, shape, e0, n, idx_d, w_d)
        _check_block(y, oracle.moe_share_rows(x, full["idx"], full["w"].astype(np.float64), experts, e0, n),
                     "%s block [%d, %d)" % (name, e0, e0 + n))
        tot += y
    assert np.abs(tot - full["y"]).max() <= PARTITION_TOL * np.abs(full["y"]).max()
    for e0, n in [(3, 5), (0, 1), (w.E - 1, 1), (1, w.E - 1)]:
        y = _share(w, t, shape, e0, n, idx_d, w_d)
        _check_block(y, oracle.moe_share_rows(x, full["idx"], full["w"].astype(np.float64), experts, e0, n),
                     "%s block [%d, %d)" % (name, e0, e0 + n))


def test_share_empty_block_and_caller_routing():
    """A caller-made routing that uses only experts 0..7 of the tiny shape: the block [8, 16)
    gets no pair and must come back exactly 0; [0, 8) is then the whole layer."""
    w = SMALL["tiny"]
    t = synth.device_inputs(w)
    shape = _shape(w)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(8)[:w.top_k] for _ in range(w.T)]).astype(np.int32)
    wt = rng.uniform(0.1, 1.0, size=idx.shape).astype(np.float32)
    idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(wt).cuda()
    assert np.all(_share(w, t, shape, 8, 8, idx_d, w_d) == 0.0)
    x = synth.hidden(w)
    experts = _experts_host(w, range(8))
    ref = oracle.moe_rows(x, idx, wt.astype(np.float64), experts, w.E)
    _check_block(_share(w, t, shape, 0, 8, idx_d, w_d), ref, "caller routing [0, 8)")


@pytest.mark.parametrize("cfg", [1, 2])
def test_share_beam_groups(cfg):
    """Beam shape: the 8 routing groups (32 experts each, one GPU's share under EP=8); the
    partition property on every token, the oracle on a token sample of two groups."""
    w = recipes.WORKLOADS[cfg]
    print("case share beam", w.name, flush=True)
    t = synth.device_inputs(w)
    shape = _shape(w)
    full = _gpu_forward(w, t, shape)
    idx_d = torch.from_numpy(full["idx"]).cuda()
    w_d = torch.from_numpy(full["w"]).cuda()
    gs = w.E // w.n_group
    ys = [_share(w, t, shape, g * gs, gs, idx_d, w_d) for g in range(w.n_group)]
    tot = np.sum(ys, axis=0, dtype=np.float64)
    err = np.abs(tot - full["y"]).max()
    print("%s: partition max|sum - y| %.3e, max|y| %.3e" % (w.name, err, np.abs(full["y"]).max()))
    assert err <= PARTITION_TOL * np.abs(full["y"]).max()
    counts = np.bincount(full["idx"].reshape(-1) // gs, minlength=w.n_group)
    x_oracle, _, _ = _oracle_inputs(w)
    for g in (0, int(np.argmax(counts))):
        e0 = g * gs
        local = (full["idx"] >= e0) & (full["idx"] < e0 + gs)
        rows = np.nonzero(local.any(axis=1))[0]
        rng = np.random.default_rng(cfg * 10 + g)
        pick = sorted(set(rng.choice(rows, size=min(6, len(rows)), replace=False).tolist()) | {0, w.T - 1})
        ids = np.unique(full["idx"][pick][local[pick]])
        ref = oracle.moe_share_rows(x_oracle[pick], full["idx"][pick], full["w"][pick].astype(np.float64),
                                    _experts_host(w, ids), e0, gs)
        err, rms = P.output_error(ys[g][pick], ref)
        print("%s group %d: %d sampled tokens, max|dy| %.3e, rms %.3e" % (w.name, g, len(pick), err, rms))
        assert np.isfinite(ys[g]).all()
        assert err <= P.Y_TOL * rms


def test_share_zero_tokens_is_noop():
    w = recipes.Workload(41, "share_T0", T=0, d=256, E=16, n_group=4, topk_group=2, top_k=4, I=128)
    shape = _shape(w)
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    assert moe.beam_moe_experts_share(shape, 0, 4, z, z, z, z, z, z, z, None, check=False) == moe.BEAM_MOE_OK
