"""The C ABI without a GPU: the library loads, exports what include/beam_moe.h
declares, and rejects bad arguments on the host before launching anything.

Every call here either fails validation or has T = 0, so no kernel is ever
launched (the fake pointers below are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_moe_layer_beam_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = (moe.BEAM_MOE_OK, moe.BEAM_MOE_ERR_INVALID_ARG,
                                      moe.BEAM_MOE_ERR_UNSUPPORTED_SHAPE, moe.BEAM_MOE_ERR_WORKSPACE_TOO_SMALL)
A = 1 << 20          # a 16-byte-aligned fake device address (never dereferenced)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(beam_moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (beam_moe_\w+)", out))
    assert set(_declared()) <= exported


def test_shape_struct_matches_header_layout():
    assert ctypes.sizeof(moe.beam_moe_shape) == 48
    assert moe.beam_moe_shape.routed_scaling_factor.offset == 32
    assert moe.beam_moe_shape.rms_eps.offset == 40
    assert moe.beam_moe_shape.weight_layout.offset == 44
    text = open(HEADER).read()
    assert "BEAM_MOE_WEIGHTS_ROW_MAJOR = 0" in text and "BEAM_MOE_WEIGHTS_PACKED = 1" in text
    assert (moe.WEIGHTS_ROW_MAJOR, moe.WEIGHTS_PACKED) == (0, 1)


def beam(T=64, **kw):
    args = dict(T=T, d=5120, E=256, n_group=8, topk_group=4, top_k=8, I=2560)
    args.update(kw)
    return moe.make_shape(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(), OK),
    (dict(T=-1), INVALID),
    (dict(d=0), INVALID),
    (dict(E=250), INVALID),            # not divisible by n_group
    (dict(topk_group=9), INVALID),
    (dict(top_k=129), INVALID),        # more than topk_group * group size
    (dict(d=5000), UNSUPPORTED),       # not a multiple of 64
    (dict(I=2500), UNSUPPORTED),
    (dict(top_k=17, topk_group=8), UNSUPPORTED),
    (dict(E=96, n_group=8), UNSUPPORTED),
    (dict(E=2048, n_group=8), UNSUPPORTED),
    (dict(E=256, n_group=256, topk_group=4, top_k=4), UNSUPPORTED),   # group of one expert
    (dict(E=256, n_group=128, topk_group=4), UNSUPPORTED),   # more than 64 groups
    (dict(E=24, n_group=4, topk_group=2, top_k=4), UNSUPPORTED),  # 6 lanes per group
    (dict(T=1 << 28), UNSUPPORTED),    # T * top_k overflows int32 pair ids
    (dict(weight_layout=1), OK),
    (dict(weight_layout=2), INVALID),
    (dict(weight_layout=-1), INVALID),
])
def test_shape_validation(kw, status):
    s = beam(**kw)
    nbytes = moe.beam_moe_workspace_bytes(s)
    assert (nbytes > 0) == (status == OK)
    st = moe.beam_moe_forward(s, A, None, A, A, A, A, A, A, None, None, None, None, stream=0, check=False)
    # with a valid shape the missing workspace is what is reported
    assert st == (INVALID if status == OK else status)


def test_workspace_size_grows_with_T_and_is_enough_for_all_entry_points():
    sizes = [moe.beam_moe_workspace_bytes(beam(T)) for T in (1, 64, 8192, 32768)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    # y_perm (T*K*d fp32) and h (T*K*I bf16) dominate the forward workspace
    assert sizes[3] >= 32768 * 8 * (5120 * 4 + 2560 * 2)


def test_null_and_misaligned_pointers_are_rejected():
    s = beam()
    n = moe.beam_moe_workspace_bytes(s)

    class WS:  # fake workspace object: only its address and byte size are read
        def __init__(self, ptr, nbytes):
            self.p, self.n = ptr, nbytes

        def data_ptr(self):
            return self.p

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    ws_small = WS(A, n - 1)
    ws_misaligned = WS(A + 8, n)
    f = lambda *a: moe.beam_moe_forward(s, *a, stream=0, check=False)
    assert f(A, None, A, A, A, A, A, A, None, None, None, ws_small) == WS_SMALL
    assert f(A, None, A, A, A, A, A, A, None, None, None, ws_misaligned) == INVALID
    assert f(None, None, A, A, A, A, A, A, None, None, None, ws_small) == INVALID      # x missing
    assert f(A, None, A, A, A, A, None, A, None, None, None, ws_small) == INVALID      # Wd missing
    assert f(A + 2, None, A, A, A, A, A, A, None, None, None, ws_small) == INVALID     # misaligned x
    assert f(A, None, A, A, A, A, A, A, A + 4, None, None, ws_small) == INVALID        # misaligned idx
    r = lambda *a: moe.beam_moe_route(s, *a, stream=0, check=False)
    assert r(A, A, None, A, A, A, A, None, ws_small) == INVALID        # norm weight without x_normed
    assert r(A, None, None, A, A, A, A, None, ws_small) == WS_SMALL
    d = lambda *a: moe.beam_moe_dispatch(s, *a, stream=0, check=False)
    assert d(A, A, None, None, ws_small) == INVALID                    # sorted_pairs missing
    assert d(A, A, A, None, ws_small) == WS_SMALL
    with pytest.raises(moe.BeamMoeError):
        moe.beam_moe_dispatch(s, A, A, A, None, ws_small, stream=0)


def test_residual_entry_points_validate_before_launching():
    s = beam()
    n = moe.beam_moe_workspace_bytes(s)

    class WS:
        def data_ptr(self):
            return A

        def numel(self):
            return n - 1

        def element_size(self):
            return 1

    ws_small = WS()
    f = lambda *a: moe.beam_moe_forward_residual(s, *a, stream=0, check=False)
    # args: x, norm_w, Wr, bias, Wg, Wu, Wd, post_w, layer, resid, resid_out, y, idx, w, logits, ws
    assert f(A, None, A, A, A, A, A, A, 3, A, A, None, None, None, None, ws_small) == WS_SMALL   # y optional
    assert f(A, None, A, A, A, A, A, None, 3, A, A, A, None, None, None, ws_small) == INVALID    # post_w missing
    assert f(A, None, A, A, A, A, A, A, -1, A, A, A, None, None, None, ws_small) == INVALID      # layer < 0
    assert f(A, None, A, A, A, A, A, A, 3, A + 4, A, A, None, None, None, ws_small) == INVALID   # misaligned resid
    assert f(A, None, A, A, A, A, A, A, 3, A, None, A, None, None, None, ws_small) == INVALID    # resid_out missing
    p = lambda sh, *a: moe.beam_moe_post_residual(sh, *a, stream=0, check=False)
    assert p(s, None, A, 3, A, A) == INVALID                                  # y missing
    assert p(s, A, A, -2, A, A) == INVALID
    assert p(beam(d=16384 + 64), A, A, 3, A, A) == UNSUPPORTED                # row longer than a block holds
    assert p(beam(T=0), A, A, 3, A, A) == OK
    assert moe.beam_moe_forward_residual(beam(T=0), A, None, A, A, A, A, A, A, 0, A, A, None, None, None, None,
                                         None, stream=0, check=False) == OK


def test_dense_mlp_validates_before_launching():
    n = moe.beam_moe_dense_workspace_bytes(64, 5120, 20480)
    assert n >= 64 * 20480 * 2
    assert moe.beam_moe_dense_workspace_bytes(-1, 5120, 20480) == 0

    class WS:
        def __init__(self, nbytes):
            self.n = nbytes

        def data_ptr(self):
            return A

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    f = lambda T, d, I, *a: moe.beam_moe_dense_mlp(T, d, I, *a, stream=0, check=False)
    assert f(64, 5120, 20480, A, A, A, A, A, WS(n - 1)) == WS_SMALL
    assert f(64, 5120, 20480, None, A, A, A, A, WS(n)) == INVALID          # x missing
    assert f(64, 5120, 20480, A, A, A, A, A + 4, WS(n)) == INVALID         # misaligned y
    assert f(65, 5120 + 64, 20480, A, A, A, A, A, WS(n)) == UNSUPPORTED    # GEMM path: d not a multiple of 128
    assert f(64, 5120 + 32, 20480, A, A, A, A, A, WS(n)) == UNSUPPORTED    # stream path: d not a multiple of 128
    assert f(64, 5120, 20480 + 64, A, A, A, A, A, WS(n)) == UNSUPPORTED    # stream path: I not a multiple of 128
    assert f(2000, 2048, 512, A, A, A, A, A, WS(n)) == UNSUPPORTED         # I below 2048 (output bar)
    assert f(64, 2048, 1920, A, A, A, A, A, WS(n)) == UNSUPPORTED          # the same on the stream path
    assert moe.beam_moe_dense_mlp(64, 5120, 20480, A, A, A, A, A, WS(n), weight_layout=2, stream=0,
                                  check=False) == INVALID
    assert f(-3, 5120, 20480, A, A, A, A, A, WS(n)) == INVALID
    assert f(1 << 20, 5120, 20480, A, A, A, A, A, WS(n)) == UNSUPPORTED   # T * I reaches 2^31
    assert f(0, 5120, 20480, A, A, A, A, A, None) == OK


def test_fp8_entry_points_validate_before_launching():
    q = lambda *a: moe.beam_moe_quantize_fp8(*a, stream=0, check=False)
    assert q(10, 48, A, A, A) == INVALID           # K not a multiple of 32
    assert q(10, 64, None, A, A) == INVALID
    assert q(10, 64, A + 2, A, A) == INVALID
    assert q(0, 64, A, A, A) == OK
    s = beam()
    n = moe.beam_moe_workspace_bytes(s)

    class WS:
        def __init__(self, nbytes):
            self.n = nbytes

        def data_ptr(self):
            return A

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    f = lambda sh, *a: moe.beam_moe_forward_fp8(sh, *a, stream=0, check=False)
    # args: x, norm_w, Wr, bias, Wg8, Wu8, Wd8, sg, su, sd, y, idx, w, logits, ws
    assert f(s, A, None, A, A, A, A, A, A, A, A, A, None, None, None, WS(n - 1)) == WS_SMALL
    assert f(s, A, None, A, A, A, A, A, A, None, A, A, None, None, None, WS(n)) == INVALID      # su missing
    big = beam(T=8192)                                                                          # prefill-sized
    assert f(big, A, None, A, A, A, A, A, A, A, A, A, None, None, None, WS(n)) == UNSUPPORTED
    odd = beam(d=5120 + 128)                                                                    # d % 512 != 0
    assert f(odd, A, None, A, A, A, A, A, A, A, A, A, None, None, None, WS(n)) == UNSUPPORTED



def test_expert_share_validates_before_launching():
    s = beam()
    n = moe.beam_moe_share_workspace_bytes(s, 32)
    assert 0 < n < moe.beam_moe_workspace_bytes(s)
    assert moe.beam_moe_share_workspace_bytes(s, 0) == 0
    assert moe.beam_moe_share_workspace_bytes(s, 257) == 0

    class WS:
        def __init__(self, nbytes):
            self.n = nbytes

        def data_ptr(self):
            return A

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    f = lambda sh, e0, ne, *a: moe.beam_moe_experts_share(sh, e0, ne, *a, stream=0, check=False)
    # args: x, idx, w, Wg, Wu, Wd, y_part, ws
    assert f(s, 0, 32, A, A, A, A, A, A, A, WS(n - 1)) == WS_SMALL
    assert f(s, 224, 33, A, A, A, A, A, A, A, WS(n)) == INVALID       # block past the last expert
    assert f(s, -1, 32, A, A, A, A, A, A, A, WS(n)) == INVALID
    assert f(s, 0, 0, A, A, A, A, A, A, A, WS(n)) == INVALID
    assert f(s, 0, 32, A, None, A, A, A, A, A, WS(n)) == INVALID      # topk_idx missing
    assert f(s, 0, 32, A, A, A, A, A, A, A + 8, WS(n)) == INVALID     # misaligned y_part
    assert f(beam(d=5120 + 32), 0, 32, A, A, A, A, A, A, A, WS(n)) == UNSUPPORTED
    assert f(beam(T=0), 0, 32, A, A, A, A, A, A, A, None) == OK


def test_pack_weights_validates_before_launching():
    f = lambda *a: moe.beam_moe_pack_weights(*a, stream=0, check=False)
    assert f(24, 64, A, A + (1 << 20)) == INVALID          # rows not a multiple of 16
    assert f(32, 48, A, A + (1 << 20)) == INVALID          # K not a multiple of 32
    assert f(32, 64, A, A) == INVALID                      # in place
    assert f(32, 64, A + 2, A + (1 << 20)) == INVALID      # misaligned
    assert f(32, 64, None, A) == INVALID
    assert f(-16, 64, A, A + (1 << 20)) == INVALID
    assert f(1 << 36, 1 << 10, A, A + (1 << 20)) == UNSUPPORTED
    assert f(0, 64, A, A + (1 << 20)) == OK


def test_fp8_packed_layout_validates_like_row_major():
    s = beam(weight_layout=1)
    n = moe.beam_moe_workspace_bytes(s)

    class WS:
        def __init__(self, nbytes):
            self.n = nbytes

        def data_ptr(self):
            return A

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    f = lambda sh, *a: moe.beam_moe_forward_fp8(sh, *a, stream=0, check=False)
    assert f(s, A, None, A, A, A, A, A, A, A, A, A, None, None, None, WS(n - 1)) == WS_SMALL
    assert f(beam(T=8192, weight_layout=1), A, None, A, A, A, A, A, A, A, A, A, None, None, None, WS(n)) == UNSUPPORTED

def test_zero_tokens_returns_ok_without_workspace():
    s = beam(T=0)
    assert moe.beam_moe_forward(s, A, None, A, A, A, A, A, A, None, None, None, None, stream=0, check=False) == OK
    assert moe.beam_moe_route(s, A, None, None, A, A, A, A, None, None, stream=0, check=False) == OK
    assert moe.beam_moe_dispatch(s, A, A, A, None, None, stream=0, check=False) == OK


def test_status_strings():
    assert moe.beam_moe_status_string(OK) == "ok"
    assert "workspace" in moe.beam_moe_status_string(WS_SMALL)
    assert moe.beam_moe_status_string(99) == "unknown status"


def test_forward_noalloc_validates_before_launching():
    """The no-allocation forward rejects bad arguments and shapes whose workspace exceeds its fixed
    64 MiB scratch before it touches the GPU (no device is needed for any of these calls)."""
    f = lambda s, *a: moe.beam_moe_forward_noalloc(s, *a, stream=0, check=False)
    args = (A, None, A, A, A, A, A, A, None, None, None)
    assert f(beam(T=512), *args) == WS_SMALL                      # 133 MiB of workspace
    assert moe.beam_moe_workspace_bytes(beam(T=192)) <= 64 << 20   # the largest Beam batch it takes
    assert f(beam(T=64), None, None, A, A, A, A, A, A, None, None, None) == INVALID     # x missing
    assert f(beam(T=64), A, None, A, A, A, A, A, A + 4, None, None, None) == INVALID    # misaligned y
    assert f(beam(T=64, d=5120 + 32), *args) == UNSUPPORTED
    assert f(beam(T=0), *args) == OK
