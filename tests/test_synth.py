"""The seeded input generator (host side): known answers, random access, laws."""
import numpy as np

import synth
from synth import recipes


def test_philox_known_answers():
    # Known-answer vectors of Philox4x32-10 published with the Random123 library
    # (Salmon et al., SC'11): counter, key -> output.
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
        ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
        ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
         [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
    ]
    for ctr, key, out in kat:
        assert list(synth.philox4x32_10(ctr, key)) == out


def test_random_access_and_determinism():
    full = synth.host_normal(200_003, 77, 4, 0.0, 0.5, synth.BF16)
    again = synth.host_normal(200_003, 77, 4, 0.0, 0.5, synth.BF16)
    assert np.array_equal(full, again)
    for start, n in [(0, 10), (1, 9), (12345, 1000), (200_000, 3)]:
        part = synth.host_normal(n, 77, 4, 0.0, 0.5, synth.BF16, start=start)
        assert np.array_equal(part, full[start:start + n])
    other = synth.host_normal(1000, 78, 4, 0.0, 0.5, synth.BF16)
    assert not np.array_equal(other, full[:1000])


def test_normal_law_moments():
    n = 1_000_000
    v = synth.host_normal(n, 5, 1, 0.0, 1.0, synth.F32).astype(np.float64)
    assert abs(v.mean()) < 5 / np.sqrt(n)
    assert abs(v.std() - 1.0) < 5 * np.sqrt(0.5 / n)
    # Kurtosis of a normal is 3.
    assert abs(((v - v.mean()) ** 4).mean() / v.var() ** 2 - 3.0) < 0.05
    w = synth.host_normal(n, 5, 1, 1.0, 0.02, synth.F32).astype(np.float64)
    assert abs(w.mean() - 1.0) < 5 * 0.02 / np.sqrt(n)


def test_uniform_law_and_bf16_rounding():
    u = synth.host_uniform(100_000, 9, 3, -0.1, 0.1, synth.F32)
    assert u.min() >= -0.1 and u.max() < 0.1
    assert abs(u.mean()) < 5 * 0.2 / np.sqrt(12 * 100_000)
    f = synth.host_normal(10_000, 3, 2, 0.0, 1.0, synth.F32)
    b = synth.host_normal(10_000, 3, 2, 0.0, 1.0, synth.BF16)
    # bf16 = float rounded to nearest even on the upper 16 bits.
    bits = f.view(np.uint32)
    exp = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(b, exp)


def test_permutation_and_hot_experts():
    p = synth.permutation(256, 1003, recipes.TID_HOT)
    assert sorted(p.tolist()) == list(range(256))
    w = recipes.WORKLOADS[3]
    hot = synth.hot_expert_ids(w)
    assert len(hot) == 16 and len(set(hot.tolist())) == 16
    b = synth.bias(w)
    assert np.all(b[hot] == np.float32(0.5))
    rest = np.setdiff1d(np.arange(256), hot)
    assert b[rest].min() >= -0.1 and b[rest].max() < 0.1


def test_workload_recipes():
    W = recipes.WORKLOADS
    assert [W[i].T for i in range(5)] == [128, 64, 8192, 4096, 32768]
    for i in (1, 2, 3, 4):
        w = W[i]
        assert (w.d, w.E, w.n_group, w.topk_group, w.top_k, w.I) == (5120, 256, 8, 4, 8, 2560)
    assert W[4].prenorm and not W[2].prenorm
    assert len({W[i].seed for i in range(5)}) == 5
