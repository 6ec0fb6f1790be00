"""Python face of the CPU oracle (libbeam_oracle.so, plain C++ in double).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline leg import this package. Nothing on the GPU path imports it, and it
imports nothing from the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILT = os.path.join(_HERE, "libbeam_oracle.so")
# BEAM_ORACLE_LIB: load another build of the same source instead (a sanitizer build, for instance)
LIB = os.environ.get("BEAM_ORACLE_LIB") or _BUILT

_c_i32p = ctypes.POINTER(ctypes.c_int32)


def build() -> None:
    cmd = ["g++", "-O3", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           os.path.join(_HERE, "beam_oracle.cpp"), "-o", _BUILT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stderr)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError("libbeam_oracle.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.oracle_bf16_round.argtypes = [vp, i64, vp]
        L.oracle_rmsnorm.argtypes = [vp, vp, i64, i32, dbl, vp, i32]
        L.oracle_logits.argtypes = [vp, vp, i64, i32, i32, vp, i32]
        L.oracle_route.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32, dbl, i32, vp, vp, vp, vp, i32]
        L.oracle_weights_for.argtypes = [vp, i64, i32, i32, vp, dbl, i32, vp]
        L.oracle_dispatch.argtypes = [vp, i64, i32, vp, vp, vp]
        L.oracle_expert.argtypes = [vp, i64, vp, vp, vp, i32, i32, vp, i32]
        L.oracle_moe_rows.argtypes = [vp, i64, vp, vp, i32, vp, vp, vp, i32, i32, vp, i32]
        L.oracle_moe_share_rows.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, i32, i32, vp, i32]
        L.oracle_post_norm.argtypes = [vp, vp, i64, i32, dbl, vp, i32]
        L.oracle_residual_step.argtypes = [vp, vp, i64, i32, vp]
        L.oracle_contribution_index.argtypes = [i32, i32]
        L.oracle_contribution_index.restype = i32
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = dbl
        L.oracle_e4m3_round.argtypes = [dbl]
        L.oracle_e4m3_round.restype = ctypes.c_uint8
        L.oracle_fp8_quantize.argtypes = [vp, i64, i32, vp, vp, i32]
        L.oracle_fp8_dequantize.argtypes = [vp, vp, i64, i32, vp]
        L.oracle_fp8_dequantize.restype = i64
        _lib = L
    return _lib


_THREADS = None


def nthreads() -> int:
    """Threads of the oracle's parallel loops: the host's cores, at most 16 (the CPU share of one
    GPU on the boxes this runs on), unless set_threads() fixed a number."""
    if _THREADS is not None:
        return _THREADS
    return max(1, min(16, os.cpu_count() or 1))


def set_threads(n) -> None:
    """Fix the oracle's thread count (None: back to the default)."""
    global _THREADS
    _THREADS = None if n is None else max(1, int(n))


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def bf16_round(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_round(v.ctypes.data, v.size, out.ctypes.data)
    return out


def rmsnorm(h: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """h [T,d] bf16 bits, w [d] bf16 bits -> x [T,d] bf16 bits."""
    h = _c(h, np.uint16)
    w = _c(w, np.uint16)
    T, d = h.shape
    x = np.empty_like(h)
    lib().oracle_rmsnorm(h.ctypes.data, w.ctypes.data, T, d, eps, x.ctypes.data, nthreads())
    return x


def logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    Wr = _c(Wr, np.float32)
    T, d = x.shape
    E = Wr.shape[1]
    z = np.empty((T, E), dtype=np.float64)
    lib().oracle_logits(x.ctypes.data, Wr.ctypes.data, T, d, E, z.ctypes.data, nthreads())
    return z


def route(x, Wr, bias, n_group, topk_group, top_k, scale, norm_topk_prob=True, want_logits=False):
    """-> idx [T,K] int32, w [T,K] float64, gap [T] float64 (and z [T,E] when asked)."""
    x = _c(x, np.uint16)
    Wr = _c(Wr, np.float32)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = Wr.shape[1]
    idx = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    gap = np.empty(T, dtype=np.float64)
    z = np.empty((T, E), dtype=np.float64) if want_logits else None
    lib().oracle_route(x.ctypes.data, Wr.ctypes.data, bias.ctypes.data, T, d, E, n_group, topk_group, top_k,
                       float(scale), int(bool(norm_topk_prob)), idx.ctypes.data, w.ctypes.data, gap.ctypes.data,
                       z.ctypes.data if z is not None else None, nthreads())
    return (idx, w, gap, z) if want_logits else (idx, w, gap)


def weights_for(z: np.ndarray, idx: np.ndarray, scale: float, norm_topk_prob=True) -> np.ndarray:
    z = _c(z, np.float64)
    idx = _c(idx, np.int32)
    T, E = z.shape
    K = idx.shape[1]
    w = np.empty((T, K), dtype=np.float64)
    lib().oracle_weights_for(z.ctypes.data, T, E, K, idx.ctypes.data, float(scale), int(bool(norm_topk_prob)),
                             w.ctypes.data)
    return w


def dispatch(idx: np.ndarray, E: int):
    """-> offsets [E+1], sorted_pairs [P], pair_rank [P] (all int32)."""
    flat = _c(idx, np.int32).reshape(-1)
    P = flat.size
    off = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(P, dtype=np.int32)
    pr = np.empty(P, dtype=np.int32)
    lib().oracle_dispatch(flat.ctypes.data, P, E, off.ctypes.data, sp.ctypes.data, pr.ctypes.data)
    return off, sp, pr


def expert(x_rows, wg, wu, wd) -> np.ndarray:
    """One expert on n rows -> o [n,d] float64."""
    x_rows = _c(x_rows, np.uint16)
    wg, wu, wd = (_c(a, np.uint16) for a in (wg, wu, wd))
    n, d = x_rows.shape
    I = wg.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lib().oracle_expert(x_rows.ctypes.data, n, wg.ctypes.data, wu.ctypes.data, wd.ctypes.data, d, I,
                        o.ctypes.data, nthreads())
    return o


def moe_rows(x_rows, idx, w, experts, E: int) -> np.ndarray:
    """Layer output for n rows with routing (idx, w); experts maps id -> (Wg[e], Wu[e], Wd[e])."""
    x_rows = _c(x_rows, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    n, d = x_rows.shape
    K = idx.shape[1]
    keep = []
    ptrs = [(ctypes.c_void_p * E)() for _ in range(3)]
    I = None
    for e in np.unique(idx):
        mats = [_c(a, np.uint16) for a in experts[int(e)]]
        keep.append(mats)
        I = mats[0].shape[0]
        for k in range(3):
            ptrs[k][int(e)] = mats[k].ctypes.data
    y = np.empty((n, d), dtype=np.float64)
    lib().oracle_moe_rows(x_rows.ctypes.data, n, idx.ctypes.data, w.ctypes.data, K, ptrs[0], ptrs[1], ptrs[2],
                          d, I, y.ctypes.data, nthreads())
    return y


def moe_share_rows(x_rows, idx, w, experts, e_begin: int, e_count: int) -> np.ndarray:
    """Expert-parallel share: the part of the layer output from experts [e_begin, e_begin+e_count)
    ("Use HF Transformers" cookbook, Parallelism). experts maps global id -> (Wg[e], Wu[e], Wd[e])
    and needs only the ids in the range that idx uses."""
    x_rows = _c(x_rows, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    n, d = x_rows.shape
    K = idx.shape[1]
    keep = []
    ptrs = [(ctypes.c_void_p * max(1, e_count))() for _ in range(3)]
    I = 1
    for e in np.unique(idx):
        if not (e_begin <= int(e) < e_begin + e_count):
            continue
        mats = [_c(a, np.uint16) for a in experts[int(e)]]
        keep.append(mats)
        I = mats[0].shape[0]
        for k in range(3):
            ptrs[k][int(e) - e_begin] = mats[k].ctypes.data
    y = np.empty((n, d), dtype=np.float64)
    lib().oracle_moe_share_rows(x_rows.ctypes.data, n, idx.ctypes.data, w.ctypes.data, K, e_begin, e_count, ptrs[0],
                                ptrs[1], ptrs[2], d, I, y.ctypes.data, nthreads())
    return y


def forward(x, Wr, bias, Wg, Wu, Wd, n_group, topk_group, top_k, scale, norm_topk_prob=True):
    """Whole layer for small problems: -> y [T,d] float64, idx, w, gap. Wg/Wu [E,I,d], Wd [E,d,I]."""
    idx, w, gap = route(x, Wr, bias, n_group, topk_group, top_k, scale, norm_topk_prob)
    E = Wr.shape[1]
    experts = {e: (Wg[e], Wu[e], Wd[e]) for e in range(E)}
    y = moe_rows(x, idx, w, experts, E)
    return y, idx, w, gap


def post_norm(y: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Post-MLP RMSNorm of y [T,d] (any float, taken as double), w [d] bf16 bits -> [T,d] float64."""
    y = _c(y, np.float64)
    w = _c(w, np.uint16)
    T, d = y.shape
    n = np.empty_like(y)
    lib().oracle_post_norm(y.ctypes.data, w.ctypes.data, T, d, float(eps), n.ctypes.data, nthreads())
    return n


def residual_step(r: np.ndarray, c: np.ndarray, k: int) -> np.ndarray:
    """Stream after adding the k-th contribution c: r*sqrt((k-1)/k) + c/sqrt(k), float64."""
    r = _c(r, np.float64)
    c = _c(c, np.float64)
    if r.shape != c.shape:
        raise ValueError("shape mismatch")
    out = np.empty_like(r)
    lib().oracle_residual_step(r.ctypes.data, c.ctypes.data, r.size, int(k), out.ctypes.data)
    return out


def contribution_index(layer: int, is_mlp: bool) -> int:
    return int(lib().oracle_contribution_index(int(layer), int(bool(is_mlp))))


def post_residual(y, w, eps, resid, layer):
    """MoE output y [T,d] -> residual stream after the MLP of 0-indexed layer `layer` (float64)."""
    k = contribution_index(layer, True)
    return residual_step(resid, post_norm(y, w, eps), k)


def e4m3_value(code: int) -> float:
    return float(lib().oracle_e4m3_value(int(code)))


def e4m3_round(v: float) -> int:
    return int(lib().oracle_e4m3_round(float(v)))


def fp8_quantize(w: np.ndarray):
    """[rows, K] bf16 bits -> (q [rows, K] uint8 E4M3 codes, s [rows, K/32] uint8 E8M0 scales)."""
    w = _c(w, np.uint16)
    rows, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    q = np.empty((rows, K), dtype=np.uint8)
    s = np.empty((rows, K // 32), dtype=np.uint8)
    lib().oracle_fp8_quantize(w.ctypes.data, rows, K, q.ctypes.data, s.ctypes.data, nthreads())
    return q, s


def fp8_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """-> [rows, K] bf16 bits of 2^(s-127) * e4m3(q); raises if any value is not exact in bf16."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    rows, K = q.shape
    out = np.empty((rows, K), dtype=np.uint16)
    bad = lib().oracle_fp8_dequantize(q.ctypes.data, s.ctypes.data, rows, K, out.ctypes.data)
    if bad:
        raise ValueError("%d dequantized values are not exact in bf16" % bad)
    return out
