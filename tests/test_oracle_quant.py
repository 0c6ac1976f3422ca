"""Pins of the oracle's NVFP4 row quantizer.

The pages name the format but print no quantizer, so the pins are hand-worked blocks
(derivations below), closed-form facts of the two-level scheme, and exact invariances.
"""
import numpy as np
import pytest

from oracle import nvfp4


def _codes(nib):
    return [int(c) for c in nvfp4.unpack_nibbles(nib)]


def test_worked_example_ascending_block():
    """x = 1..16.  amax = 16, gs = 16/2688.  The only block has bmax = amax, so
    sf = 16 / (6 * gs) = 448 -> scale byte 0x7E, and d = 448 * gs = 8/3 (float32
    2.6666667).  x/d = 0.375, 0.75, 1.125, 1.5, 1.875, 2.25, 2.625, 3, 3.375, 3.75,
    4.125, 4.5, 4.875, 5.25, 5.625, 6.  Nearest e2m1 with ties to even (0.75 sits
    exactly between 0.5 and 1.0 in float32 and goes to 1.0, code 2):
    1,2,2,3,4,4,5,5,5,6,6,6,6,7,7,7."""
    nib, sc, gs = nvfp4.quantize_row(np.arange(1, 17, dtype=np.float32))
    assert _codes(nib) == [1, 2, 2, 3, 4, 4, 5, 5, 5, 6, 6, 6, 6, 7, 7, 7]
    assert list(sc) == [0x7E]
    assert gs == np.float32(16.0) / np.float32(2688.0)
    assert nib[0] == 0x21            # even element in the low nibble


def test_worked_example_signed_block():
    """x = -8..7.  amax = 8, d = 448 * 8/2688 = 4/3.  x/d = -6, -5.25, -4.5, -3.75, -3,
    -2.25, -1.5, -0.75, 0, 0.75, 1.5, 2.25, 3, 3.75, 4.5, 5.25 -> codes
    F,F,E,E,D,C,B,A,0,2,3,4,5,6,6,7 (-0.75 and 0.75 are ties that go to 1.0)."""
    nib, sc, gs = nvfp4.quantize_row(np.arange(-8, 8, dtype=np.float32))
    assert _codes(nib) == [0xF, 0xF, 0xE, 0xE, 0xD, 0xC, 0xB, 0xA,
                           0x0, 0x2, 0x3, 0x4, 0x5, 0x6, 0x6, 0x7]
    assert list(sc) == [0x7E]


def test_worked_example_ties_and_signed_zero():
    """amax = 6 so d = 448 * 6/2688 = 1 and x/d = x.  Ties: 0.25 -> 0 (code 0),
    0.75 -> 1.0 (code 2), 2.5 -> 2.0 (code 4); -0.1875 rounds to zero and keeps its
    sign (0x8); -0.0 stays 0x8."""
    x = np.array([6, 3, 1.5, 0.75, 0.375, 0.1875, 0, -6, -3, -1.5, -0.75, -0.375,
                  -0.1875, -0.0, 0.25, 2.5], dtype=np.float32)
    nib, sc, gs = nvfp4.quantize_row(x)
    assert _codes(nib) == [0x7, 0x5, 0x3, 0x2, 0x1, 0x0, 0x0, 0xF,
                           0xD, 0xB, 0xA, 0x9, 0x8, 0x8, 0x0, 0x4]


def test_zero_row_and_zero_block():
    nib, sc, gs = nvfp4.quantize_row(np.zeros(64, dtype=np.float32))
    assert not nib.any() and not sc.any() and gs == 1.0
    x = np.zeros(48, dtype=np.float32)
    x[16:32] = np.linspace(-3, 3, 16, dtype=np.float32)
    x[40] = -0.0
    nib, sc, gs = nvfp4.quantize_row(x)
    codes = _codes(nib)
    assert sc[0] == 0 and sc[2] == 0 and sc[1] == 0x7E
    assert codes[:16] == [0] * 16 and codes[32:] == [0] * 16   # d == 0 -> plain 0x0


def test_tiny_block_underflows_to_zero_scale():
    # a block 2^-12 times smaller than the row max needs a scale of 448 * 2^-12 ~ 0.11:
    # fine; a block 2^-20 smaller needs ~4e-4 < 2^-10 and underflows to scale 0
    x = np.zeros(48, dtype=np.float32)
    x[0] = 1.0
    x[16] = 2.0 ** -12
    x[32] = 2.0 ** -20
    nib, sc, gs = nvfp4.quantize_row(x)
    assert sc[1] != 0 and sc[2] == 0
    assert _codes(nib)[32] == 0


def test_block_holding_amax_gets_max_scale():
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = rng.standard_normal(256).astype(np.float32) * np.float32(rng.uniform(0.01, 100))
        nib, sc, gs = nvfp4.quantize_row(x)
        k = int(np.argmax(np.abs(x)))
        assert sc[k // 16] == 0x7E
        assert _codes(nib)[k] & 7 == 7                      # |x| / d rounds to 6


@pytest.mark.parametrize("p", [-20, -3, 1, 7, 30])
def test_power_of_two_scaling_is_exact(p):
    """Multiplying a row by 2^p scales gs by 2^p and leaves every code and block scale
    unchanged (every step is a float32 op that commutes with exact power-of-two
    scaling, as long as nothing under- or overflows)."""
    rng = np.random.default_rng(p + 100)
    x = rng.standard_normal(512).astype(np.float32)
    n0, s0, g0 = nvfp4.quantize_row(x)
    n1, s1, g1 = nvfp4.quantize_row(x * np.float32(2.0 ** p))
    assert np.array_equal(n0, n1) and np.array_equal(s0, s1)
    assert g1 == g0 * np.float32(2.0 ** p)


def test_reconstruction_error_bound():
    """Each element is within half an e2m1 step (of its block's grid) of x/d, except
    above 6 where it saturates; d = e4m3(sf) * gs is within 1/16 of bmax/6."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(4096) * np.exp(rng.uniform(-4, 4, 4096))).astype(np.float32)
    nib, sc, gs = nvfp4.quantize_row(x)
    codes = np.array(_codes(nib))
    val = nvfp4.e2m1_decode(codes) * np.repeat(nvfp4.e4m3_decode(sc), 16) * float(gs)
    d = np.repeat(nvfp4.e4m3_decode(sc), 16) * float(gs)
    ratio = np.abs(x.astype(np.float64)) / d
    half_gap = np.where(ratio <= 2, 0.25, np.where(ratio <= 4, 0.5, 1.0))
    err = np.abs(val - x) / d
    ok = (err <= half_gap * (1 + 1e-6)) | (ratio > 6)
    assert ok.all()
    xb = np.abs(x.astype(np.float64)).reshape(-1, 16).max(1)
    dd = nvfp4.e4m3_decode(sc) * float(gs)
    assert np.all(np.abs(dd - xb / 6) <= xb / 6 / 16 + 1e-30)


def test_rows_are_independent():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((5, 128)).astype(np.float32)
    q, s, g = nvfp4.quantize_rows(X)
    for i in range(5):
        qi, si, gi = nvfp4.quantize_row(X[i])
        assert np.array_equal(q[i], qi) and np.array_equal(s[i], si) and g[i] == gi


def _exhaustive_nearest(v, table):
    """Index of the value of `table` (ascending magnitudes, code = index) nearest to |v|
    by exact rational comparison, ties to the even index, saturating at the last entry."""
    from fractions import Fraction
    a = abs(Fraction(float(v)))
    best, best_d = 0, None
    for i, t in enumerate(table):
        d = abs(Fraction(float(t)) - a)
        if best_d is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


@pytest.mark.parametrize("rows", [1, 130])
def test_quantizer_against_exhaustive_search(rows):
    """The page's test shape (K = 64, one row and 130 rows of random values spanning many
    binades): every scale byte and every element code equals the one found by searching
    the whole e4m3 / e2m1 code tables with exact rational distances, applied to the
    float32 quotients of the stated formulas."""
    rng = np.random.default_rng(64 + rows)
    x = (rng.standard_normal((rows, 64)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    x[0, 5] = -0.0
    e2_pos = nvfp4.e2m1_decode(np.arange(8))
    e4_pos = nvfp4.e4m3_decode(np.arange(0x7F))
    for r in range(rows):
        nib, sc, gs = nvfp4.quantize_row(x[r])
        codes = nvfp4.unpack_nibbles(nib)
        amax = np.float32(np.max(np.abs(x[r])))
        assert gs == (np.float32(amax / np.float32(2688.0)) if amax > 0 else np.float32(1.0))
        for b in range(4):
            blk = x[r, 16 * b:16 * (b + 1)]
            sf = np.float32(np.max(np.abs(blk)) / np.float32(np.float32(6.0) * gs))
            want_sc = _exhaustive_nearest(sf, e4_pos)
            assert sc[b] == want_sc, (r, b)
            d = np.float32(np.float32(e4_pos[want_sc]) * gs)
            for k in range(16):
                got = int(codes[16 * b + k])
                if d == 0:
                    assert got == 0
                    continue
                q = np.float32(blk[k] / d)
                want = _exhaustive_nearest(q, e2_pos) | (8 if np.signbit(q) else 0)
                assert got == want, (r, b, k, float(q))
