"""Independent helpers used by the tests to pin the oracle: numpy/torch library
routines, textbook roundings and exhaustive enumeration. None of this code is
shared with the oracle or with the GPU path."""
from __future__ import annotations

import itertools
import math

import numpy as np


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits_rne(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even (8 significant bits).

    Written from the definition with numpy's frexp/ldexp and its half-to-even
    rint, so it shares nothing with the oracle's rounding routine."""
    v = np.asarray(v, dtype=np.float64)
    m, ex = np.frexp(v)                     # v = m * 2^ex, 0.5 <= |m| < 1
    step = np.maximum(ex - 8, -133)
    q = np.rint(np.ldexp(v, -step))         # rint rounds half to even
    r = np.ldexp(q, step).astype(np.float32)  # exact: <= 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def brute_route_token(z_row, bias, G, KG, K, S, norm=True):
    """Group-limited top-K by exhaustive enumeration (small shapes only).

    group score = the largest b[i] + b[j] over distinct experts i, j of the group;
    kept groups = the KG-subset of groups with the largest total score;
    chosen experts = the K-subset of candidates with the largest total b.
    Returns (sorted expert ids, {id: weight})."""
    E = len(z_row)
    gsz = E // G
    s = sigmoid(np.asarray(z_row, dtype=np.float64))
    b = s + np.asarray(bias, dtype=np.float64)
    gs = []
    for g in range(G):
        mem = range(g * gsz, (g + 1) * gsz)
        gs.append(max(b[i] + b[j] for i, j in itertools.combinations(mem, 2)))
    best_groups = max(itertools.combinations(range(G), KG), key=lambda c: sum(gs[g] for g in c))
    cand = [e for g in best_groups for e in range(g * gsz, (g + 1) * gsz)]
    best = max(itertools.combinations(cand, K), key=lambda c: sum(b[e] for e in c))
    tot = sum(s[e] for e in best)
    w = {e: (S * s[e] / tot if norm else S * s[e]) for e in best}
    return sorted(best), w


def comb(n, k):
    return math.comb(n, k)
