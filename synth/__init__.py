"""Seeded synthetic input generator shared by the oracle side and the GPU side.

It holds no arithmetic of the MoE layer: only the counter-based generator
(Philox4x32-10) and the value laws of the workloads. `libsynth_host.so` fills
host arrays; `libsynth_dev.so` fills device memory with bit-identical values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .recipes import (WORKLOADS, Workload, DENSE_WORKLOADS, DenseWorkload, TID_X, TID_WR, TID_BIAS, TID_WG, TID_WU, TID_WD,
                      TID_H, TID_NORMW, TID_HOT, TID_RESID, TID_POSTW)

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_BUILT = os.path.join(_HERE, "libsynth_host.so")
# BEAM_SYNTH_HOST_LIB: load another build of synth_host.c instead (a sanitizer build, for instance)
HOST_LIB = os.environ.get("BEAM_SYNTH_HOST_LIB") or _HOST_BUILT
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

F32, BF16 = 0, 1


def build(verbose: bool = False) -> None:
    """Compile the host generator (gcc) and the device generator (hipcc, gfx950)."""
    cmds = [
        ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
         os.path.join(_HERE, "synth_host.c"), "-o", _HOST_BUILT, "-lm"],
        [HIPCC, "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         os.path.join(_HERE, "synth_dev.hip"), "-o", DEV_LIB],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("synth build failed: %s\n%s" % (" ".join(c), r.stderr))
        if verbose and r.stderr:
            print(r.stderr)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError("libsynth_host.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        i64, u64, u32, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, i64, i64, u64, u32, dbl, dbl, ctypes.c_int]
        lib.synth_fill_uniform.argtypes = [ctypes.c_void_p, ctypes.c_int, i64, i64, u64, u32, dbl, dbl, ctypes.c_int]
        lib.synth_permutation.argtypes = [ctypes.c_void_p, ctypes.c_int32, u64, u32]
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError("libsynth_dev.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        i64, u64, u32, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double
        for fn in (lib.synth_dev_fill_normal, lib.synth_dev_fill_uniform):
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int, i64, i64, u64, u32, dbl, dbl, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        _dev = lib
    return _dev


def _nthreads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    _host_lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def host_normal(n: int, seed: int, tid: int, mean: float, std: float, dtype: int, start: int = 0,
                out: np.ndarray | None = None) -> np.ndarray:
    """Elements start..start+n of a normal stream; bf16 comes back as uint16 bit patterns."""
    if out is None:
        out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    assert out.flags.c_contiguous and out.size == n
    _host_lib().synth_fill_normal(out.ctypes.data, dtype, start, n, seed, tid, mean, std, _nthreads())
    return out


def host_uniform(n: int, seed: int, tid: int, lo: float, hi: float, dtype: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    _host_lib().synth_fill_uniform(out.ctypes.data, dtype, start, n, seed, tid, lo, hi, _nthreads())
    return out


def permutation(n: int, seed: int, tid: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _host_lib().synth_permutation(out.ctypes.data, n, seed, tid)
    return out


def dev_normal(ptr: int, n: int, seed: int, tid: int, mean: float, std: float, dtype: int,
               start: int = 0, stream: int = 0) -> None:
    rc = _dev_lib().synth_dev_fill_normal(ptr, dtype, start, n, seed, tid, mean, std, stream)
    if rc != 0:
        raise RuntimeError("synth_dev_fill_normal failed (%d)" % rc)


def dev_uniform(ptr: int, n: int, seed: int, tid: int, lo: float, hi: float, dtype: int,
                start: int = 0, stream: int = 0) -> None:
    rc = _dev_lib().synth_dev_fill_uniform(ptr, dtype, start, n, seed, tid, lo, hi, stream)
    if rc != 0:
        raise RuntimeError("synth_dev_fill_uniform failed (%d)" % rc)


# ---------------------------------------------------------------------------------------------
# Workload tensors on the host (numpy). Small tensors are always made here.

def bias(w: Workload) -> np.ndarray:
    """Per-expert bias: U(lo, hi), and `hot_bias` on the first `hot_experts` of a seeded shuffle."""
    b = host_uniform(w.E, w.seed, TID_BIAS, w.bias_lo, w.bias_hi, F32)
    if w.hot_experts:
        b[hot_expert_ids(w)] = np.float32(w.hot_bias)
    return b


def hot_expert_ids(w: Workload) -> np.ndarray:
    if not w.hot_experts:
        return np.zeros(0, dtype=np.int32)
    return np.sort(permutation(w.E, w.seed, TID_HOT)[: w.hot_experts])


def router_weight(w: Workload) -> np.ndarray:
    """Wr, [d, E] fp32, N(0, 1/sqrt(d))."""
    return host_normal(w.d * w.E, w.seed, TID_WR, 0.0, w.std_in, F32).reshape(w.d, w.E)


def hidden(w: Workload, rows=None) -> np.ndarray:
    """x (or the pre-norm h for prenorm workloads), [T, d] bf16 bits; optional row subset."""
    tid = TID_H if w.prenorm else TID_X
    if rows is None:
        return host_normal(w.T * w.d, w.seed, tid, 0.0, 1.0, BF16).reshape(w.T, w.d)
    out = np.empty((len(rows), w.d), dtype=np.uint16)
    for i, r in enumerate(rows):
        host_normal(w.d, w.seed, tid, 0.0, 1.0, BF16, start=int(r) * w.d, out=out[i])
    return out


def norm_weight(w: Workload) -> np.ndarray:
    """Pre-MLP RMSNorm weight, [d] bf16 bits, N(1, 0.02)."""
    return host_normal(w.d, w.seed, TID_NORMW, 1.0, 0.02, BF16)


def post_norm_weight(w: Workload) -> np.ndarray:
    """Post-MLP RMSNorm weight, [d] bf16 bits, N(1, 0.02)."""
    return host_normal(w.d, w.seed, TID_POSTW, 1.0, 0.02, BF16)


def residual(w: Workload) -> np.ndarray:
    """Residual stream before the MLP's contribution, [T, d] fp32, N(0, 1) (the depth-scaled
    residual keeps the stream at unit scale)."""
    return host_normal(w.T * w.d, w.seed, TID_RESID, 0.0, 1.0, F32).reshape(w.T, w.d)


def expert_weights(w: Workload, e: int):
    """(Wg[e] [I, d], Wu[e] [I, d], Wd[e] [d, I]) as bf16 bits, generated on the host."""
    n = w.I * w.d
    wg = host_normal(n, w.seed, TID_WG, 0.0, w.std_in, BF16, start=e * n).reshape(w.I, w.d)
    wu = host_normal(n, w.seed, TID_WU, 0.0, w.std_in, BF16, start=e * n).reshape(w.I, w.d)
    wd = host_normal(n, w.seed, TID_WD, 0.0, w.std_down, BF16, start=e * n).reshape(w.d, w.I)
    return wg, wu, wd


# ---------------------------------------------------------------------------------------------
# Workload tensors on the GPU (torch tensors; the generator kernels run on the current stream).

def device_inputs(w: Workload, device="cuda"):
    """All inputs of one workload, resident in HBM. Big tensors are made on the GPU."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    t = {}
    hid = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=device)
    dev_normal(hid.data_ptr(), hid.numel(), w.seed, TID_H if w.prenorm else TID_X, 0.0, 1.0, BF16, stream=stream)
    if w.prenorm:
        t["h"] = hid
        t["norm_w"] = torch.from_numpy(norm_weight(w).view(np.int16)).view(torch.bfloat16).to(device)
    else:
        t["x"] = hid
    t["Wr"] = torch.from_numpy(router_weight(w)).to(device)
    t["bias"] = torch.from_numpy(bias(w)).to(device)
    n = w.E * w.I * w.d
    for name, tid, std, shape in (("Wg", TID_WG, w.std_in, (w.E, w.I, w.d)),
                                  ("Wu", TID_WU, w.std_in, (w.E, w.I, w.d)),
                                  ("Wd", TID_WD, w.std_down, (w.E, w.d, w.I))):
        ten = torch.empty(shape, dtype=torch.bfloat16, device=device)
        dev_normal(ten.data_ptr(), n, w.seed, tid, 0.0, std, BF16, stream=stream)
        t[name] = ten
    return t


# ---------------------------------------------------------------------------------------------
# Dense SwiGLU MLP workloads.

def dense_hidden(w: DenseWorkload, rows=None) -> np.ndarray:
    """x, [T, d] bf16 bits (optionally only the given rows)."""
    if rows is None:
        return host_normal(w.T * w.d, w.seed, TID_X, 0.0, 1.0, BF16).reshape(w.T, w.d)
    out = np.empty((len(rows), w.d), dtype=np.uint16)
    for i, r in enumerate(rows):
        host_normal(w.d, w.seed, TID_X, 0.0, 1.0, BF16, start=int(r) * w.d, out=out[i])
    return out


def dense_weights(w: DenseWorkload):
    """(Wg [I, d], Wu [I, d], Wd [d, I]) as bf16 bits, generated on the host."""
    n = w.I * w.d
    wg = host_normal(n, w.seed, TID_WG, 0.0, w.std_in, BF16).reshape(w.I, w.d)
    wu = host_normal(n, w.seed, TID_WU, 0.0, w.std_in, BF16).reshape(w.I, w.d)
    wd = host_normal(n, w.seed, TID_WD, 0.0, w.std_down, BF16).reshape(w.d, w.I)
    return wg, wu, wd


def dense_device_inputs(w: DenseWorkload, device="cuda"):
    """x, Wg, Wu, Wd of a dense workload generated in HBM (same values as the host twins)."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    t = {}
    for name, tid, std, shape in (("x", TID_X, 1.0, (w.T, w.d)), ("Wg", TID_WG, w.std_in, (w.I, w.d)),
                                  ("Wu", TID_WU, w.std_in, (w.I, w.d)), ("Wd", TID_WD, w.std_down, (w.d, w.I))):
        ten = torch.empty(shape, dtype=torch.bfloat16, device=device)
        dev_normal(ten.data_ptr(), ten.numel(), w.seed, tid, 0.0, std, BF16, stream=stream)
        t[name] = ten
    return t
