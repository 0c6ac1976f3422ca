"""Pins of the oracle's NVFP4 codec against facts that do not come from the oracle.

* The OCP 8-bit / 4-bit float definitions, written out as value tables by hand.
* The pages' e4m3 fold probe ([MF] "Different globals on the two halves").
* Round-to-nearest-even checked on every midpoint of both grids, enumerated here.
* A brute-force nearest search by linear scan, a different route from the oracle's.
"""
import os

import numpy as np
import pytest

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


# e2m1 magnitudes of codes 0..7 as listed by the OCP MX format definition
E2M1_BY_HAND = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_matches_definition():
    for c in range(8):
        assert nvfp4.e2m1_decode_scalar(c) == E2M1_BY_HAND[c]
        neg = nvfp4.e2m1_decode_scalar(c | 8)
        assert neg == -E2M1_BY_HAND[c] and np.signbit(neg)


def test_e2m1_step_near_one_is_fifty_percent():
    # [MF] "Different globals on the two halves": NVFP4's e2m1 step is 50% near 1.0
    grid = sorted(set(abs(v) for v in nvfp4.E2M1_TABLE))
    i = grid.index(1.0)
    assert (grid[i + 1] - grid[i]) / grid[i] == 0.5


def test_e4m3fn_landmarks():
    t = nvfp4.E4M3_TABLE
    finite_pos = [b for b in range(256) if np.isfinite(t[b]) and t[b] > 0]
    assert len(finite_pos) == 126          # [MF]: "all 126 finite positive e4m3 codes"
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x7E] == 448.0                # largest finite
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0
    assert t[0x39] == 1.125
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0xB8] == -1.0
    # strictly increasing over the positive finite codes (monotone encoding)
    assert np.all(np.diff(t[0x00:0x7F]) > 0)


def test_encode_decode_roundtrip_every_code():
    for c in range(16):
        assert nvfp4.e2m1_encode(nvfp4.e2m1_decode(c)) == c
    for b in range(256):
        if b in (0x7F, 0xFF):
            continue
        assert nvfp4.e4m3_encode(nvfp4.e4m3_decode(b)) == b


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_every_midpoint_goes_to_even_code(fmt):
    if fmt == "e2m1":
        vals, enc, top = nvfp4.E2M1_TABLE[:8], nvfp4.e2m1_encode, 7
    else:
        vals, enc, top = nvfp4.E4M3_TABLE[:0x7F], nvfp4.e4m3_encode, 0x7E
    for c in range(top):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2                 # exact in float64 (few significant bits)
        even = c if c % 2 == 0 else c + 1
        assert enc(mid) == even, (fmt, c, mid)
        assert enc(-mid) == (even | (0x8 if fmt == "e2m1" else 0x80))
        assert enc(np.nextafter(mid, 0)) == c
        assert enc(np.nextafter(mid, np.inf)) == c + 1


def test_saturation():
    assert nvfp4.e2m1_encode(6.5) == 7 and nvfp4.e2m1_encode(1e30) == 7
    assert nvfp4.e2m1_encode(-100.0) == 0xF
    assert nvfp4.e4m3_encode(449.0) == 0x7E and nvfp4.e4m3_encode(1e30) == 0x7E
    assert nvfp4.e4m3_encode(np.inf) == 0x7E
    assert nvfp4.e4m3_encode(-500.0) == 0xFE


def test_underflow_and_signed_zero():
    assert nvfp4.e4m3_encode(2.0 ** -11) == 0x00          # below half the smallest subnormal
    assert nvfp4.e4m3_encode(2.0 ** -10) == 0x00          # exact tie with 0 -> even (0)
    assert nvfp4.e4m3_encode(np.nextafter(2.0 ** -10, 1)) == 0x01
    assert nvfp4.e2m1_encode(-0.0) == 0x8
    assert nvfp4.e2m1_encode(-0.1) == 0x8
    assert nvfp4.e2m1_encode(0.25) == 0x0                  # tie with 0 -> even (0)


def _scan_nearest(v, table, codes):
    best = None
    for c in codes:
        d = abs(abs(v) - table[c])
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_brute_force_nearest_random():
    rng = np.random.default_rng(1)
    n = 3000
    mags = np.exp2(rng.uniform(-12, 10, n))
    vals = mags * rng.choice([-1.0, 1.0], n)
    enc4 = nvfp4.e4m3_encode(vals)
    enc2 = nvfp4.e2m1_encode(vals / 64.0)
    for k in range(n):
        v = vals[k]
        want = _scan_nearest(v, nvfp4.E4M3_TABLE, range(0x7F)) | (0x80 if v < 0 else 0)
        assert enc4[k] == want, v
        w2 = vals[k] / 64.0
        want2 = _scan_nearest(w2, nvfp4.E2M1_TABLE, range(8)) | (0x8 if w2 < 0 else 0)
        assert enc2[k] == want2, w2


def test_fold_probe_reproduces_page_statistics():
    """[MF] "Different globals on the two halves", option (b): fold the gate/up global
    ratio into every finite positive e4m3 code and re-encode."""
    g = _read_golden("fold_probe.txt")
    ratio = g["gate_global"] / g["up_global"]
    assert round(ratio, 4) == g["ratio_printed"]
    codes = [b for b in range(0x7F) if nvfp4.E4M3_TABLE[b] > 0]
    assert len(codes) == g["finite_positive_codes"]
    v = nvfp4.e4m3_decode(codes) * ratio
    q = nvfp4.e4m3_decode(nvfp4.e4m3_encode(v))
    rel = np.abs(q - v) / v
    assert abs(rel.mean() * 100 - g["mean_rel_err_pct"]) < 0.005
    assert abs(rel.max() * 100 - g["max_rel_err_pct"]) < 0.005
    assert int(np.sum(v > 448.0)) == g["saturated_codes"]
    assert np.all(q[v > 448.0] == 448.0)                          # saturated, not NaN


def test_bf16_rounding_against_float32_cases():
    # values exactly representable in float32: bf16 RNE equals the classic bit rounding
    rng = np.random.default_rng(2)
    f = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    bits = f.view(np.uint32).astype(np.uint64)
    want = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    got = nvfp4.f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rounding_float64_ties_and_double_rounding():
    # 1 + 2^-8 is the exact midpoint between bf16 1.0 and 1.0078125: ties to even (1.0)
    assert nvfp4.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80
    # a hair above the midpoint rounds up, even though float32 would round it back to
    # the midpoint first (a double-rounding trap)
    assert nvfp4.f64_to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert nvfp4.f64_to_bf16_bits(-2.0) == 0xC000
    assert nvfp4.f64_to_bf16_bits(0.0) == 0x0000
    assert nvfp4.f64_to_bf16_bits(3.4e38) == 0x7F80        # above max: overflows to inf
    assert nvfp4.f64_to_bf16_bits(2.0 ** -133) == 0x0001   # smallest subnormal


def test_every_element_scale_product_is_exact_in_bf16_and_every_pair_in_fp32():
    """The exactness the GEMMs rely on: an e2m1 value times an e4m3fn scale has at most
    2 + 4 significant bits and stays inside bf16's exponent range, so every such product
    (all 16 element codes x all 254 finite scale codes) is a bf16 value; and the product
    of two of them has at most 12 significant bits, so it is exact in fp32.  Checked by
    rounding each product to bf16 / fp32 and comparing with the float64 value."""
    e2 = nvfp4.e2m1_decode(np.arange(16))
    s8 = nvfp4.e4m3_decode(np.array([b for b in range(256) if b not in (0x7F, 0xFF)]))
    assert len(s8) == 254 and np.isfinite(s8).all()
    prods = np.unique(np.outer(e2, s8).ravel())
    back = nvfp4.bf16_bits_to_f32(nvfp4.f64_to_bf16_bits(prods)).astype(np.float64)
    assert np.array_equal(back, prods)
    mags = np.unique(np.abs(prods[prods != 0]))
    pairs = np.outer(mags, mags)                  # exact in float64 (<= 12 significant bits)
    assert np.array_equal(pairs.astype(np.float32).astype(np.float64), pairs)
    assert pairs.min() > 0 and pairs.max() < np.finfo(np.float32).max
