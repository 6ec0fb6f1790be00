"""Python binding of libbeam_moe.so: one Beam sparse-MoE layer forward on MI355X.

Argument marshalling only. Every step of the layer runs in the library's HIP
kernels; the entry points take torch device tensors (or raw device pointers as
ints) and queue work on the current torch stream unless one is given. The
contract of each call is in include/beam_moe.h.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# BEAM_MOE_LIB: load another build of the same sources instead (a host-sanitizer build, for instance)
LIB_PATH = os.environ.get("BEAM_MOE_LIB") or os.path.join(_PKG, "libbeam_moe.so")

BEAM_MOE_OK = 0
BEAM_MOE_ERR_INVALID_ARG = 1
BEAM_MOE_ERR_UNSUPPORTED_SHAPE = 2
BEAM_MOE_ERR_WORKSPACE_TOO_SMALL = 3
BEAM_MOE_ERR_HIP = 4

EXPORTED = ("beam_moe_workspace_bytes", "beam_moe_route", "beam_moe_dispatch", "beam_moe_forward",
            "beam_moe_forward_staged", "beam_moe_post_residual", "beam_moe_forward_residual",
            "beam_moe_dense_workspace_bytes", "beam_moe_dense_mlp", "beam_moe_quantize_fp8",
            "beam_moe_forward_fp8", "beam_moe_share_workspace_bytes", "beam_moe_experts_share",
            "beam_moe_pack_weights", "beam_moe_forward_noalloc", "beam_moe_status_string")
N_STAGE_EVENTS = 6


class beam_moe_shape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("norm_topk_prob", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("weight_layout", ctypes.c_int32),
    ]


class BeamMoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, beam_moe_status_string(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libbeam_moe.so is missing: build it with __graft_entry__.build() "
                               "(the MoE layer has no non-HIP implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        shp = ctypes.POINTER(beam_moe_shape)
        L.beam_moe_workspace_bytes.argtypes = [shp]
        L.beam_moe_workspace_bytes.restype = sz
        L.beam_moe_route.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_route.restype = i32
        L.beam_moe_dispatch.argtypes = [shp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_dispatch.restype = i32
        L.beam_moe_forward.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_forward.restype = i32
        L.beam_moe_forward_staged.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.beam_moe_forward_staged.restype = i32
        L.beam_moe_post_residual.argtypes = [shp, vp, vp, i32, vp, vp, vp]
        L.beam_moe_post_residual.restype = i32
        L.beam_moe_forward_residual.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                                vp, sz, vp, vp]
        L.beam_moe_forward_residual.restype = i32
        L.beam_moe_dense_workspace_bytes.argtypes = [ctypes.c_int64, i32, i32]
        L.beam_moe_dense_workspace_bytes.restype = sz
        L.beam_moe_dense_mlp.argtypes = [ctypes.c_int64, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_dense_mlp.restype = i32
        L.beam_moe_quantize_fp8.argtypes = [ctypes.c_int64, i32, vp, vp, vp, vp]
        L.beam_moe_quantize_fp8.restype = i32
        L.beam_moe_forward_fp8.argtypes = [shp] + [vp] * 14 + [sz, vp, vp]
        L.beam_moe_forward_fp8.restype = i32
        L.beam_moe_share_workspace_bytes.argtypes = [shp, i32]
        L.beam_moe_share_workspace_bytes.restype = sz
        L.beam_moe_experts_share.argtypes = [shp, i32, i32] + [vp] * 7 + [vp, sz, vp, vp]
        L.beam_moe_experts_share.restype = i32
        L.beam_moe_pack_weights.argtypes = [ctypes.c_int64, i32, vp, vp, vp]
        L.beam_moe_pack_weights.restype = i32
        L.beam_moe_forward_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.beam_moe_forward_noalloc.restype = i32
        L.beam_moe_status_string.argtypes = [i32]
        L.beam_moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


WEIGHTS_ROW_MAJOR, WEIGHTS_PACKED = 0, 1


def make_shape(T, d, E, n_group, topk_group, top_k, I, routed_scaling_factor=2.5, norm_topk_prob=True,
               rms_eps=1e-6, weight_layout=WEIGHTS_ROW_MAJOR) -> beam_moe_shape:
    return beam_moe_shape(int(T), int(d), int(E), int(n_group), int(topk_group), int(top_k), int(I),
                          float(routed_scaling_factor), int(bool(norm_topk_prob)), float(rms_eps),
                          int(weight_layout))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    if t is None:
        return 0
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> int:
    if status != BEAM_MOE_OK:
        raise BeamMoeError(status, where)
    return status


def beam_moe_status_string(status: int) -> str:
    return lib().beam_moe_status_string(int(status)).decode()


def beam_moe_workspace_bytes(shape: beam_moe_shape) -> int:
    return int(lib().beam_moe_workspace_bytes(ctypes.byref(shape)))


def beam_moe_route(shape, x, norm_w, x_normed, Wr, bias, topk_idx, topk_w, logits, workspace, stream=None,
                   check=True) -> int:
    st = lib().beam_moe_route(ctypes.byref(shape), _ptr(x), _ptr(norm_w), _ptr(x_normed), _ptr(Wr), _ptr(bias),
                              _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(workspace), _nbytes(workspace),
                              _stream(stream))
    return _check(st, "beam_moe_route") if check else st


def beam_moe_dispatch(shape, topk_idx, expert_offsets, sorted_pairs, pair_rank, workspace, stream=None,
                      check=True) -> int:
    st = lib().beam_moe_dispatch(ctypes.byref(shape), _ptr(topk_idx), _ptr(expert_offsets), _ptr(sorted_pairs),
                                 _ptr(pair_rank), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return _check(st, "beam_moe_dispatch") if check else st


def beam_moe_forward(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, workspace, stream=None,
                     check=True) -> int:
    st = lib().beam_moe_forward(ctypes.byref(shape), _ptr(x), _ptr(norm_w), _ptr(Wr), _ptr(bias), _ptr(Wg),
                                _ptr(Wu), _ptr(Wd), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                                _ptr(workspace), _nbytes(workspace), _stream(stream))
    return _check(st, "beam_moe_forward") if check else st


def beam_moe_forward_noalloc(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, stream=None,
                             check=True) -> int:
    """beam_moe_forward on the library's fixed per-GPU scratch (no workspace argument, no allocation)."""
    st = lib().beam_moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(norm_w), _ptr(Wr), _ptr(bias), _ptr(Wg),
                                        _ptr(Wu), _ptr(Wd), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                                        _stream(stream))
    return _check(st, "beam_moe_forward_noalloc") if check else st


def beam_moe_forward_staged(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, y, topk_idx, topk_w, logits, workspace,
                            stage_events, stream=None, check=True) -> int:
    """stage_events: sequence of N_STAGE_EVENTS hipEvent_t handles (ints) or None entries."""
    arr = None
    if stage_events is not None:
        arr = (ctypes.c_void_p * N_STAGE_EVENTS)(*[e if e else None for e in stage_events])
    st = lib().beam_moe_forward_staged(ctypes.byref(shape), _ptr(x), _ptr(norm_w), _ptr(Wr), _ptr(bias), _ptr(Wg),
                                       _ptr(Wu), _ptr(Wd), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                                       _ptr(workspace), _nbytes(workspace), _stream(stream), arr)
    return _check(st, "beam_moe_forward_staged") if check else st


def _events(stage_events):
    if stage_events is None:
        return None
    return (ctypes.c_void_p * N_STAGE_EVENTS)(*[e if e else None for e in stage_events])


def beam_moe_post_residual(shape, y, post_w, layer, resid, resid_out, stream=None, check=True) -> int:
    st = lib().beam_moe_post_residual(ctypes.byref(shape), _ptr(y), _ptr(post_w), int(layer), _ptr(resid),
                                      _ptr(resid_out), _stream(stream))
    return _check(st, "beam_moe_post_residual") if check else st


def beam_moe_forward_residual(shape, x, norm_w, Wr, bias, Wg, Wu, Wd, post_w, layer, resid, resid_out, y, topk_idx,
                              topk_w, logits, workspace, stage_events=None, stream=None, check=True) -> int:
    st = lib().beam_moe_forward_residual(ctypes.byref(shape), _ptr(x), _ptr(norm_w), _ptr(Wr), _ptr(bias), _ptr(Wg),
                                         _ptr(Wu), _ptr(Wd), _ptr(post_w), int(layer), _ptr(resid), _ptr(resid_out),
                                         _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(workspace),
                                         _nbytes(workspace), _stream(stream), _events(stage_events))
    return _check(st, "beam_moe_forward_residual") if check else st


def beam_moe_dense_workspace_bytes(T: int, d: int, I: int) -> int:
    return int(lib().beam_moe_dense_workspace_bytes(int(T), int(d), int(I)))


def beam_moe_dense_mlp(T, d, I, x, Wg, Wu, Wd, y, workspace, weight_layout=WEIGHTS_ROW_MAJOR, stream=None,
                       check=True) -> int:
    st = lib().beam_moe_dense_mlp(int(T), int(d), int(I), int(weight_layout), _ptr(x), _ptr(Wg), _ptr(Wu), _ptr(Wd),
                                  _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return _check(st, "beam_moe_dense_mlp") if check else st


def beam_moe_quantize_fp8(rows, K, w, q, scales, stream=None, check=True) -> int:
    st = lib().beam_moe_quantize_fp8(int(rows), int(K), _ptr(w), _ptr(q), _ptr(scales), _stream(stream))
    return _check(st, "beam_moe_quantize_fp8") if check else st


def beam_moe_forward_fp8(shape, x, norm_w, Wr, bias, Wg8, Wu8, Wd8, sg, su, sd, y, topk_idx, topk_w, logits,
                         workspace, stage_events=None, stream=None, check=True) -> int:
    st = lib().beam_moe_forward_fp8(ctypes.byref(shape), _ptr(x), _ptr(norm_w), _ptr(Wr), _ptr(bias), _ptr(Wg8),
                                    _ptr(Wu8), _ptr(Wd8), _ptr(sg), _ptr(su), _ptr(sd), _ptr(y), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(logits), _ptr(workspace), _nbytes(workspace),
                                    _stream(stream), _events(stage_events))
    return _check(st, "beam_moe_forward_fp8") if check else st


def beam_moe_share_workspace_bytes(shape, e_count: int) -> int:
    return int(lib().beam_moe_share_workspace_bytes(ctypes.byref(shape), int(e_count)))


def beam_moe_experts_share(shape, e_begin, e_count, x, topk_idx, topk_w, Wg, Wu, Wd, y_part, workspace,
                           stage_events=None, stream=None, check=True) -> int:
    st = lib().beam_moe_experts_share(ctypes.byref(shape), int(e_begin), int(e_count), _ptr(x), _ptr(topk_idx),
                                      _ptr(topk_w), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(y_part), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream), _events(stage_events))
    return _check(st, "beam_moe_experts_share") if check else st


def beam_moe_pack_weights(rows, K, w, packed, stream=None, check=True) -> int:
    st = lib().beam_moe_pack_weights(int(rows), int(K), _ptr(w), _ptr(packed), _stream(stream))
    return _check(st, "beam_moe_pack_weights") if check else st


def pack_expert_weights(Wg, Wu, Wd, stream=None):
    """Packed copies of the expert weights (torch tensors [E, I, d], [E, I, d], [E, d, I])."""
    out = []
    for w in (Wg, Wu, Wd):
        p = w.new_empty(w.shape)
        beam_moe_pack_weights(w.shape[0] * w.shape[1], w.shape[2], w, p, stream)
        out.append(p)
    return tuple(out)


def pack_dense_weights(Wg, Wu, Wd, stream=None):
    """Packed copies of the dense MLP weights (torch tensors [I, d], [I, d], [d, I])."""
    out = []
    for w in (Wg, Wu, Wd):
        p = w.new_empty(w.shape)
        beam_moe_pack_weights(w.shape[0], w.shape[1], w, p, stream)
        out.append(p)
    return tuple(out)
