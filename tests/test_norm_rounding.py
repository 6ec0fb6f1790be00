"""The pre-MLP RMSNorm's FP32 shortcut (router.hip, norm_to_bf16) against the FP64 rounding it
stands in for, on the host: a model of the rule in numpy (float32 arithmetic rounds every
product) checked on random and on deliberately near-midpoint products. The rule: with
p = (a * float(r)) * w in FP32, take bf16(p) when p's exponent field is neither 0 nor 255 and
its low 16 bits are at least 8 ulps from the bf16 rounding midpoint 0x8000; otherwise round
(a * r) * w in FP64. Whenever the rule takes the FP32 result it must equal the FP64 one (the
Transformers "Beam" page, Overview: FP32 RMSNorm note; the FP64 product is the reading that
makes the GPU's x equal the oracle's bit for bit)."""
import numpy as np


def _bf16_bits(v32):
    u = v32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _f64_to_bf16(v64):
    """Single rounding of doubles to bf16 (round to nearest even): through round-to-odd float."""
    t = v64.astype(np.float32)                       # nearest, may round away from v64
    t64 = t.astype(np.float64)
    # truncate toward zero: step back one float where rounding went past v64 in magnitude
    over = np.abs(t64) > np.abs(v64)
    tu = t.view(np.uint32).copy()
    tu[over] -= 1
    t = tu.view(np.float32)
    inexact = t.astype(np.float64) != v64
    tu = t.view(np.uint32) | inexact.astype(np.uint32)
    return _bf16_bits(tu.view(np.float32))


def _rule(a_bits, w_bits, r):
    a = (a_bits.astype(np.uint32) << 16).view(np.float32)
    w = (w_bits.astype(np.uint32) << 16).view(np.float32)
    r = np.asarray(r, dtype=np.float64)
    r32 = r.astype(np.float32)
    p = (a * r32) * w                                # float32: each product rounded
    u = p.view(np.uint32)
    ex = (u >> 23) & 0xFF
    dist = (u & 0xFFFF).astype(np.int64) - 0x8000
    fast = (ex != 0) & (ex != 0xFF) & (np.abs(dist) >= 8)
    exact = _f64_to_bf16((a.astype(np.float64) * r) * w.astype(np.float64))
    return fast, _bf16_bits(p), exact


def test_f64_to_bf16_model_is_single_rounding():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))
    got = _f64_to_bf16(v)
    # reference: exact rounding of the double to 8 significand bits, ties to even
    m, e = np.frexp(v)                               # v = m * 2^e, 0.5 <= |m| < 1
    q = m * 256.0
    fl = np.floor(q)
    frac = q - fl
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(fl, 2) == 1))
    ref = np.ldexp((fl + up) / 256.0, e).astype(np.float32)
    assert np.array_equal(got, (ref.view(np.uint32) >> 16).astype(np.uint16))


def test_fp32_shortcut_equals_fp64_rounding():
    rng = np.random.default_rng(11)
    n = 2_000_000
    a = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for r in (0.7311243923, 1.0, 1.0 / np.sqrt(3.0), 12.3456789012345, 1e-3 + 1e-12):
        fast, p_bf, exact = _rule(a, w, r)
        # r = 1: a * w is exact in FP32 and often a bf16 midpoint itself, which FP64 then decides
        assert fast.mean() > (0.9 if r == 1.0 else 0.99), (r, fast.mean())
        assert np.array_equal(p_bf[fast], exact[fast]), r


def test_fp32_shortcut_near_midpoints():
    """Products placed within a few FP32 ulps of bf16 midpoints (r chosen per element, as the rule
    must hold for any r): the rule must send every one it cannot decide to FP64, and the ones it
    keeps must still round as FP64 does."""
    rng = np.random.default_rng(17)
    n = 400000
    a = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    af = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # target products: a bf16 midpoint plus an offset of -12..12 FP32 ulps, with the signs of a w
    mag = np.abs(rng.standard_normal(n)).astype(np.float32) + np.float32(0.01)
    mu = (mag.view(np.uint32) & 0xFFFF0000) | 0x8000
    off = rng.integers(-12, 13, n).astype(np.int64)
    tgt = (mu.astype(np.int64) + off).astype(np.uint32).view(np.float32).astype(np.float64)
    tgt *= np.sign(af * wf)
    ok = (af != 0) & (wf != 0)
    r = np.where(ok, tgt / np.where(ok, af * wf, 1.0), 1.0)
    fast, p_bf, exact = _rule(a, w, r)
    assert (~fast).sum() > 0.3 * n                   # most land inside the margin: the slow path runs
    assert fast.sum() > 0.2 * n
    assert np.array_equal(p_bf[fast], exact[fast])
