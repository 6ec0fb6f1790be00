"""Comparison rules between the GPU path and the oracle.

Routing: index sets must match exactly, except on tokens where the oracle's score
gap at a selection boundary is below EPS; such a token is "excused" when the GPU's
set is itself an EPS-optimal group-limited top-k (checked here by enumerating every
admissible group subset). Weights: 1e-5 relative. Outputs: max|dy| <= 1e-2 * rms(y_ref)
over the compared tokens; excused tokens are left out of the output comparison,
since their expected output depends on which of the near-equal choices was made.
"""
from __future__ import annotations

import itertools

import numpy as np

EPS = 1e-5
W_RTOL = 1e-5
Y_TOL = 1e-2


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def eps_optimal(z_row, bias, sel, G, KG, K, eps=EPS) -> bool:
    """Is `sel` a valid group-limited top-K within eps (any admissible kept-group set)?"""
    E = len(z_row)
    gsz = E // G
    b = sigmoid(np.asarray(z_row, np.float64)) + np.asarray(bias, np.float64)
    gs = np.array([np.sort(b[g * gsz:(g + 1) * gsz])[-2:].sum() for g in range(G)])
    kth = np.sort(gs)[::-1][KG - 1]
    sel = set(int(e) for e in sel)
    if len(sel) != K:
        return False
    for kept in itertools.combinations(range(G), KG):
        if min(gs[list(kept)]) < kth - eps:
            continue
        members = [e for g in kept for e in range(g * gsz, (g + 1) * gsz)]
        if not sel.issubset(members):
            continue
        rest = [e for e in members if e not in sel]
        if not rest or min(b[list(sel)]) >= max(b[rest]) - eps:
            return True
    return False


def compare_routing(idx_gpu, w_gpu, idx_ref, w_ref, gap, z_ref, bias, G, KG, K):
    """Returns the boolean mask of tokens whose routing matched exactly; raises on a
    mismatch that is not excused."""
    T = idx_gpu.shape[0]
    same = np.all(np.sort(idx_gpu, 1) == np.sort(idx_ref, 1), axis=1)
    bad = np.nonzero(~same)[0]
    for t in bad:
        assert gap[t] < EPS, "token %d: routing differs with oracle gap %.3e >= %g" % (t, gap[t], EPS)
        assert eps_optimal(z_ref[t], bias, idx_gpu[t], G, KG, K), "token %d: GPU set is not eps-optimal" % t
    # weights on matched tokens, compared per expert id
    m = np.nonzero(same)[0]
    og = np.argsort(idx_gpu[m], 1)
    orf = np.argsort(idx_ref[m], 1)
    wg = np.take_along_axis(w_gpu[m].astype(np.float64), og, 1)
    wr = np.take_along_axis(w_ref[m], orf, 1)
    rel = np.abs(wg - wr) / np.abs(wr)
    assert rel.max() <= W_RTOL, "routing weights: max rel err %.3e" % rel.max()
    # order: descending biased score (allowing FP32 noise)
    b = sigmoid(z_ref) + bias.astype(np.float64)[None, :]
    bsel = np.take_along_axis(b, idx_gpu.astype(np.int64), 1)
    assert np.all(np.diff(bsel, axis=1) <= EPS), "topk_idx not in descending biased-score order"
    assert np.all((idx_gpu >= 0) & (idx_gpu < z_ref.shape[1]))
    assert all(len(set(r)) == K for r in idx_gpu.tolist())
    return same


def output_error(y_gpu, y_ref):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref).max()
    rms = np.sqrt((y_ref ** 2).mean())
    return err, rms


def segment_blocks(idx_ref, E, block):
    """(expert, block) of every pair, in the expert-major stable order the dispatch defines:
    pair p = t*K + j sits at rank r inside its expert's segment and in block r // block.
    Returns (token of each pair, key of each pair, rank of each pair)."""
    flat = np.asarray(idx_ref, np.int64).reshape(-1)
    K = idx_ref.shape[1]
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.empty_like(order)
    rank[order] = np.arange(len(order)) - starts[flat[order]]
    key = flat * (1 << 20) + rank // block
    return np.arange(len(flat)) // K, key, rank


def cover_tokens(idx_ref, E, block, tails=True):
    """Tokens such that every (expert, block of `block` consecutive rows of its segment) holds
    at least one of them, plus (tails) the token of each expert's last row: every work item of
    a grouped GEMM whose m-tiles are multiples of `block` rows then computes at least one
    compared output row, the ragged last tile of every expert included. Greedy set cover: each
    token covers the K blocks of its K pairs."""
    tok, key, rank = segment_blocks(idx_ref, E, block)
    K = idx_ref.shape[1]
    picks = set()
    if tails:
        flat = np.asarray(idx_ref, np.int64).reshape(-1)
        counts = np.bincount(flat, minlength=E)
        last = np.nonzero(rank == counts[flat] - 1)[0]
        picks.update(int(t) for t in tok[last])
    covered = set()
    for t in picks:
        covered.update(int(k) for k in key[t * K:(t + 1) * K])
    # for each uncovered block (in key order) take its token that covers the most uncovered blocks
    members = {}
    for p, k in enumerate(key.tolist()):
        members.setdefault(k, []).append(int(tok[p]))
    for k in sorted(members):
        if k in covered:
            continue
        best = max(members[k], key=lambda t: sum(int(q) not in covered for q in key[t * K:(t + 1) * K]))
        picks.add(best)
        covered.update(int(q) for q in key[best * K:(best + 1) * K])
    assert covered == set(members)
    return np.array(sorted(picks), dtype=np.int64)


def sample_tokens(idx_ref, n_extra=6, seed=0, must=()):
    """Deterministic token sample: first, last, tokens of the busiest expert, random others."""
    T = idx_ref.shape[0]
    rng = np.random.default_rng(seed)
    counts = np.bincount(idx_ref.reshape(-1), minlength=int(idx_ref.max()) + 1)
    busiest = int(np.argmax(counts))
    on_busiest = np.nonzero(np.any(idx_ref == busiest, axis=1))[0]
    picks = {0, T - 1}
    picks.update(int(t) for t in on_busiest[:2])
    picks.update(int(t) for t in must)
    picks.update(int(t) for t in rng.choice(T, size=min(n_extra, T), replace=False))
    return np.array(sorted(picks), dtype=np.int64)
