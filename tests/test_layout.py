"""CPU check of the test-side packing helper against the element formula in qvae.h."""
import numpy as np

from tests.layout import pack_weight_codes


def test_pack_weight_codes_matches_header_formula():
    rng = np.random.default_rng(0)
    Co, kt, kh, kw, Ci = 64, 3, 3, 3, 96
    plain = rng.integers(-127, 128, (Co, kt, kh, kw, Ci)).astype(np.int8)
    packed = pack_weight_codes(plain)
    assert packed.shape == (Co // 32, kt, Ci // 32, kh, kw, 64, 16)
    for _ in range(2000):
        cb, i, s, j, l, L, b = (rng.integers(0, m) for m in (Co // 32, kt, Ci // 32, kh, kw, 64, 16))
        assert packed[cb, i, s, j, l, L, b] == plain[32 * cb + L % 32, i, j, l, 32 * s + 16 * (L // 32) + b]
    # a permutation: every code appears exactly once
    assert np.array_equal(np.sort(packed.ravel()), np.sort(plain.ravel()))


def test_pack_weights_bf16_matches_header_formula():
    from tests.layout import pack_weights_bf16
    rng = np.random.default_rng(1)
    Co, Ci, kt, kh, kw = 64, 48, 3, 3, 3
    w = rng.integers(0, 1 << 16, (Co, Ci, kt, kh, kw)).astype(np.uint16)
    packed = pack_weights_bf16(w)
    assert packed.shape == (Co // 32, kt, Ci // 16, kh, kw, 64, 8)
    for _ in range(2000):
        cb, i, s, j, l, L, e = (rng.integers(0, m) for m in (Co // 32, kt, Ci // 16, kh, kw, 64, 8))
        assert packed[cb, i, s, j, l, L, e] == w[32 * cb + L % 32, 16 * s + 8 * (L // 32) + e, i, j, l]
    assert np.array_equal(np.sort(packed.ravel()), np.sort(w.ravel()))
