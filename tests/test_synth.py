"""The seeded input generator: determinism, stream independence, and the workload's
distributions (code ranges, scale/bias ranges, bf16 rounding, normal moments)."""
import numpy as np
import pytest

import synth


def test_splitmix64_reference_values():
    """splitmix64 seeded with 0 yields the published first outputs of the sequence."""
    assert synth.word(0, 0) == 0xE220A8397B1DCDAF
    assert synth.word(0, 1) == 0x6E789E6AA1B965F4
    assert synth.word(0, 2) == 0x06C45D188009454F


def test_deterministic_and_independent():
    a = synth.qmat(42, 0, 1, synth.T_GATE, 4, 64, 256)
    b = synth.qmat(42, 0, 1, synth.T_GATE, 4, 64, 256)
    c = synth.qmat(42, 0, 2, synth.T_GATE, 4, 64, 256)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scale, b.scale)
    assert not np.array_equal(a.codes, c.codes)
    # any sub-block regenerates on its own: the first rows of a bigger draw are the same draw
    big = synth.codes(synth.stream(42, 0, 1, synth.T_GATE), 4, 128, 256)
    assert np.array_equal(big[:64], a.codes)


@pytest.mark.parametrize("bits", [4, 2])
def test_distributions(bits):
    q = synth.qmat(42, 1, 7, synth.T_UP, bits, 1024, 4096)
    lo, hi, bmul, spread = synth.DIST[bits]
    assert q.codes.max() == (1 << bits) - 1 and q.codes.min() == 0
    hist = np.bincount(q.codes.ravel(), minlength=1 << bits) / q.codes.size
    assert np.abs(hist - 1.0 / (1 << bits)).max() < 0.002
    s = (q.scale.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = (q.bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = 2.0 ** -8
    assert s.min() >= lo * (1 - ulp) and s.max() <= hi * (1 + ulp)
    ratio = -b / (bmul * s)
    assert ratio.min() >= (1 - spread) * (1 - 2 * ulp) and ratio.max() <= (1 + spread) * (1 + 2 * ulp)


def test_normal_moments():
    x = synth.normal(synth.stream(1, 2, 3, 4), 1 << 20, 0.02)
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 1e-4
    assert x.dtype == np.float32


def test_q2_fields():
    """2-bit codes are the 2-bit fields of the words, least significant first."""
    key = synth.stream(5, 0, 0, 1)
    c = synth.codes(key, 2, 1, 64).ravel()
    w0, w1 = synth.word(key, 0), synth.word(key, 1)
    assert [int(v) for v in c[:32]] == [(w0 >> (2 * i)) & 3 for i in range(32)]
    assert [int(v) for v in c[32:]] == [(w1 >> (2 * i)) & 3 for i in range(32)]
