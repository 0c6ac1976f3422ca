"""Pins of the oracle's layer steps: grouping, gather, grouped GEMM, SwiGLU, scatter, layer.

Each pin comes from outside the oracle: a brute-force scan, exact rational arithmetic,
reductions to a gather, known constants of the logistic function, or the invariants
the pages test ([GG] "Proof": row invariance, fused w13 == separate, determinism).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe, nvfp4

# --------------------------------------------------------------------------- grouping


def _brute_group(a_expert, a_src, a_dst, E, S, T):
    """Counting-sort by scanning experts in order and assignments in order."""
    rows = []
    for e in range(E):
        for j in range(len(a_expert)):
            if a_expert[j] == e and 0 <= a_src[j] < S and 0 <= a_dst[j] < T:
                rows.append(j)
    return rows


@pytest.mark.parametrize("seed", range(6))
def test_group_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    E, S, T, R = 7, 9, 5, 40
    a_expert = rng.integers(-1, E + 1, R)
    a_src = rng.integers(-1, S + 1, R)
    a_dst = rng.integers(0, T + 1, R)
    a_w = rng.random(R).astype(np.float32)
    g = moe.group_rows(a_expert, a_src, a_dst, a_w, E, S, T)
    rows = _brute_group(a_expert, a_src, a_dst, E, S, T)
    Rv = len(rows)
    assert g["offsets"][E] == Rv and g["offsets"][0] == 0
    assert list(g["row_src"][:Rv]) == [a_src[j] for j in rows]
    assert list(g["row_dst"][:Rv]) == [a_dst[j] for j in rows]
    assert list(g["row_w"][:Rv]) == [a_w[j] for j in rows]
    for e in range(E):
        seg = g["row_expert"][g["offsets"][e]:g["offsets"][e + 1]]
        assert np.all(seg == e)
        assert g["offsets"][e + 1] - g["offsets"][e] == sum(
            1 for j in rows if a_expert[j] == e)
    assert np.all(g["row_src"][Rv:] == -1) and np.all(g["row_w"][Rv:] == 0)
    # error bits
    want_err = 0
    if np.any((a_expert < 0) | (a_expert >= E)):
        want_err |= moe.ERR_EXPERT
    if np.any((a_src < 0) | (a_src >= S)):
        want_err |= moe.ERR_SRC
    if np.any((a_dst < 0) | (a_dst >= T)):
        want_err |= moe.ERR_DST
    assert g["err"] == want_err
    # token CSR: each token's rows ascending, covering exactly the valid rows
    seen = []
    for t in range(T):
        lst = list(g["tok_rows"][g["tok_off"][t]:g["tok_off"][t + 1]])
        assert lst == sorted(lst)
        assert all(g["row_dst"][i] == t for i in lst)
        seen += lst
    assert sorted(seen) == list(range(Rv))


def test_gather_exact_and_dropped_rows_zero():
    x = np.arange(12, dtype=np.uint16).reshape(3, 4) + 0x3F00
    out = moe.gather_rows(x, np.array([2, 0, -1, 2]))
    assert np.array_equal(out[0], x[2]) and np.array_equal(out[1], x[0])
    assert not out[2].any() and np.array_equal(out[3], x[2])


# --------------------------------------------------------------------------- GEMM
E2M1_HAND = [0, 1, 2, 3, 4, 6, 8, 12]      # 2 * e2m1 magnitude, codes 0..7


def _val(nib_row, sc_row, k):
    """Exact value of element k of an NVFP4 row, decoded by hand (no oracle code)."""
    byte = int(nib_row[k // 2])
    code = (byte >> 4) if k % 2 else (byte & 0xF)
    mag = Fraction(E2M1_HAND[code & 7], 2)
    s = int(sc_row[k // 16])
    e, m = (s >> 3) & 15, s & 7
    scale = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    if s & 0x80:
        scale = -scale
    return (-mag if code & 8 else mag) * scale


def _rand_nvfp4(rng, rows, K, scale_lo=0x00, scale_hi=0x7E):
    nib = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    sc = rng.integers(scale_lo, scale_hi + 1, (rows, K // 16)).astype(np.uint8)
    return nib, sc


def test_grouped_gemm_exact_against_rational_brute_force():
    """K <= 256: every product and partial sum is exact in float64 (exponent span of the
    products is 43 bits, +8 bits of sum), so the oracle must equal exact rationals."""
    rng = np.random.default_rng(11)
    E, N, K = 3, 5, 64
    offsets = np.array([0, 2, 2, 5])             # expert 1 is empty
    aq, as_ = _rand_nvfp4(rng, 5, K)
    W = [_rand_nvfp4(rng, N, K) for _ in range(E)]
    acc = moe.grouped_gemm(aq, as_, offsets, lambda e: W[e], N, K)
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                s = sum(_val(aq[i], as_[i], k) * _val(W[e][0][n], W[e][1][n], k)
                        for k in range(K))
                assert Fraction(acc[i, n]) == s, (e, i, n)


def test_grouped_gemm_one_hot_weights_is_a_gather():
    """Weight row n holds a single 1.0 (code 2, scale 0x38) at column perm[n]: the GEMM
    returns the activation's value at that column."""
    rng = np.random.default_rng(12)
    N = K = 32
    perm = rng.permutation(K)
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[np.arange(N), perm] = 2
    nib = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sc = np.full((N, K // 16), 0x38, np.uint8)
    aq, as_ = _rand_nvfp4(rng, 3, K, 0x20, 0x50)
    acc = moe.grouped_gemm(aq, as_, np.array([0, 3]), lambda e: (nib, sc), N, K)
    for i in range(3):
        for n in range(N):
            assert Fraction(acc[i, n]) == _val(aq[i], as_[i], perm[n])


def test_fused_w13_equals_separate_and_row_invariance():
    """[GG] "Proof": the fused gate|up operand gives the gate-only and up-only results,
    and a row's output does not depend on which rows share its group."""
    rng = np.random.default_rng(13)
    I, K = 16, 256
    gate = _rand_nvfp4(rng, I, K)
    up = _rand_nvfp4(rng, I, K)
    fused = (np.concatenate([gate[0], up[0]]), np.concatenate([gate[1], up[1]]))
    aq, as_ = _rand_nvfp4(rng, 4, K)
    off = np.array([0, 4])
    f = moe.grouped_gemm(aq, as_, off, lambda e: fused, 2 * I, K)
    g = moe.grouped_gemm(aq, as_, off, lambda e: gate, I, K)
    u = moe.grouped_gemm(aq, as_, off, lambda e: up, I, K)
    assert np.array_equal(f[:, :I], g) and np.array_equal(f[:, I:], u)
    for i in range(4):
        alone = moe.grouped_gemm(aq[i:i + 1], as_[i:i + 1], np.array([0, 1]),
                                 lambda e: fused, 2 * I, K)
        assert np.array_equal(alone[0], f[i])


# --------------------------------------------------------------------------- SwiGLU
SIGMOID_1 = 0.7310585786300049     # 1 / (1 + e^-1)
SIGMOID_2 = 0.8807970779778823
SIGMOID_3 = 0.9525741268224334


def _swiglu_one(gate, up, g_gate=1.0, g_up=1.0, gs=1.0):
    acc = np.array([[gate, up]], dtype=np.float64)
    h = moe.swiglu(acc, np.array([0, 1]), np.array([g_gate]), np.array([g_up]),
                   np.array([gs], np.float32), 1)
    return nvfp4.bf16_bits_to_f32(h)[0, 0]


def _bf16(v):
    return nvfp4.bf16_bits_to_f32(nvfp4.f64_to_bf16_bits(v))


def test_swiglu_known_values_and_halves():
    assert _swiglu_one(0.0, 5.0) == 0.0                        # silu(0) = 0
    assert _swiglu_one(1.0, 1.0) == _bf16(SIGMOID_1)
    assert _swiglu_one(2.0, 3.0) == _bf16(3 * 2 * SIGMOID_2)   # silu on the gate half
    assert _swiglu_one(3.0, 2.0) == _bf16(2 * 3 * SIGMOID_3)   # ... not on the up half
    assert _swiglu_one(40.0, 0.5) == 20.0                      # silu(z) -> z
    v = _swiglu_one(-40.0, 1.0)
    assert v < 0 and abs(v) < 1e-15                            # silu(z) -> 0-


def test_swiglu_globals_apply_per_half():
    """[MF] "Different globals on the two halves", option (a): the gate global scales the
    gate half, the up global the up half, and the row global both."""
    assert _swiglu_one(1.0, 1.0, g_gate=2.0, g_up=1.0) == _bf16(2 * SIGMOID_2)
    assert _swiglu_one(1.0, 1.0, g_gate=1.0, g_up=2.0) == _bf16(2 * SIGMOID_1)
    assert _swiglu_one(0.5, 0.5, gs=2.0) == _bf16(SIGMOID_1)


# --------------------------------------------------------------------------- scatter
def test_scatter_single_row_exact_and_empty_token():
    y = np.array([[1.0, -3.0, 0.25], [5.0, 6.0, 7.0]])
    offsets = np.array([0, 1, 2])
    row_w = np.array([0.5, 0.25], np.float32)
    g_down = np.array([2.0, 4.0], np.float32)
    gs = np.array([4.0, 0.5], np.float32)
    tok_off = np.array([0, 1, 1, 2])                 # token 1 has no rows
    tok_rows = np.array([0, 1])
    out = nvfp4.bf16_bits_to_f32(moe.scatter_add(y, offsets, row_w, g_down, gs, tok_off,
                                                 tok_rows, 3))
    assert list(out[0]) == [4.0, -12.0, 1.0]          # 0.5*2*4 * y[0]
    assert not out[1].any()
    assert list(out[2]) == [2.5, 3.0, 3.5]            # 0.25*4*0.5 * y[1]


def test_scatter_is_linear_on_exact_values():
    rng = np.random.default_rng(3)
    y1 = rng.integers(-8, 8, (4, 6)).astype(np.float64)
    y2 = rng.integers(-8, 8, (4, 6)).astype(np.float64)
    args = (np.array([0, 2, 4]), np.array([1, 0.5, 2, 1], np.float32),
            np.array([1, 2], np.float32), np.ones(4, np.float32),
            np.array([0, 3, 4]), np.array([0, 1, 3, 2]), 2)
    f = lambda y: nvfp4.bf16_bits_to_f32(moe.scatter_add(y, *args)).astype(np.float64)
    assert np.array_equal(f(y1 + y2), f(y1) + f(y2))


# --------------------------------------------------------------------------- layer
def _tiny_layer_inputs(seed, T=6, E=4, H=64, I=32, k=2):
    rng = np.random.default_rng(seed)
    W13 = [_rand_nvfp4(rng, 2 * I, H, 0x18, 0x38) for _ in range(E)]
    W2 = [_rand_nvfp4(rng, H, I, 0x18, 0x38) for _ in range(E)]
    x = nvfp4.f64_to_bf16_bits(rng.standard_normal((T, H)))
    a_expert = np.concatenate([rng.choice(E, k, replace=False) for _ in range(T)])
    a_src = np.repeat(np.arange(T), k)
    a_w = rng.random(T * k).astype(np.float32)
    gl = lambda v: np.full(E, v, np.float32)
    return dict(x=x, a_expert=a_expert, a_src=a_src, a_dst=a_src.copy(), a_w=a_w,
                W13=W13, W2=W2, g=(gl(4.65e-5), gl(3.78e-5), gl(4.2e-5)), E=E, H=H, I=I, k=k)


def _run(d, sel=None):
    T = d["x"].shape[0]
    idx = np.arange(len(d["a_expert"])) if sel is None else sel
    return moe.layer_forward(d["x"], d["a_expert"][idx], d["a_src"][idx], d["a_dst"][idx],
                             d["a_w"][idx], T, lambda e: d["W13"][e], lambda e: d["W2"][e],
                             *d["g"], d["E"], d["H"], d["I"])


def test_layer_batch_parity_and_determinism():
    """[GG] "Proof" (batch parity, five repeated calls): a token's output computed in a
    batch equals its output computed with only its own rows; repeated calls agree."""
    d = _tiny_layer_inputs(21)
    full = _run(d)
    for _ in range(2):
        assert np.array_equal(_run(d), full)
    k = d["k"]
    for t in (0, 3, 5):
        alone = _run(d, np.arange(t * k, t * k + k))
        assert np.array_equal(alone[t], full[t])
        assert not np.delete(alone, t, axis=0).any()


def test_layer_output_scale_is_sane():
    """Output ~ sum_k w * g_down * (quantized h) . w2; nonzero and finite."""
    d = _tiny_layer_inputs(22)
    out = nvfp4.bf16_bits_to_f32(_run(d))
    assert np.all(np.isfinite(out)) and np.abs(out).max() > 0


# --------------------------------------------------------------------------- W4A16
def _bf16_rows(rng, R, K, lo_exp=-1, hi_exp=1):
    """bf16 bit patterns of random values +-(1 + m/128) * 2^e, e in [lo_exp, hi_exp]."""
    m = rng.integers(0, 128, (R, K))
    e = rng.integers(lo_exp, hi_exp + 1, (R, K))
    sign = rng.integers(0, 2, (R, K))
    return ((sign << 15) | ((e + 127) << 7) | m).astype(np.uint16)


def _bf16_val(bits):
    """Exact value of a bf16 bit pattern, decoded by hand (normal numbers)."""
    b = int(bits)
    e, m = (b >> 7) & 0xFF, b & 0x7F
    v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -v if b & 0x8000 else v


def test_w4a16_gemm_exact_against_rational_brute_force():
    """K <= 256 with activation exponents in [-1, 1]: the products span < 40 bits, so the
    float64 oracle must equal the exact rational sums of bf16 x NVFP4 products."""
    rng = np.random.default_rng(31)
    E, N, K = 3, 4, 64
    offsets = np.array([0, 1, 1, 4])             # expert 1 is empty
    a = _bf16_rows(rng, 4, K)
    W = [_rand_nvfp4(rng, N, K) for _ in range(E)]
    acc = moe.grouped_gemm_w4a16(a, offsets, lambda e: W[e], N, K)
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                s = sum(_bf16_val(a[i, k]) * _val(W[e][0][n], W[e][1][n], k) for k in range(K))
                assert Fraction(acc[i, n]) == s, (e, i, n)


def test_w4a16_gemm_one_hot_activation_reads_back_a_weight_column():
    """x = 1.0 at column k only: acc[n] is the NVFP4 weight value w(n, k), decoded by hand."""
    rng = np.random.default_rng(32)
    N, K = 8, 64
    W = _rand_nvfp4(rng, N, K)
    cols = [0, 17, 63]
    a = np.zeros((len(cols), K), np.uint16)
    a[np.arange(len(cols)), cols] = 0x3F80              # bf16 1.0
    acc = moe.grouped_gemm_w4a16(a, np.array([0, len(cols)]), lambda e: W, N, K)
    for i, k in enumerate(cols):
        for n in range(N):
            assert Fraction(acc[i, n]) == _val(W[0][n], W[1][n], k)


def test_w4a16_equals_w4a4_on_activations_nvfp4_represents_exactly():
    """When each activation is exactly an NVFP4 value with row global 1 (a code times a
    power-of-two block scale), the two arithmetics meet: W4A16 over those bf16 values equals
    W4A4 over the same codes (two independently pinned GEMMs)."""
    rng = np.random.default_rng(33)
    N, K, R = 6, 128, 3
    codes = rng.integers(0, 16, (R, K)).astype(np.uint8)
    sc = rng.integers(0x30, 0x40, (R, K // 16)).astype(np.uint8) & 0x78   # powers of two
    aq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    vals = nvfp4.dequantize(aq, sc)
    bits = nvfp4.f64_to_bf16_bits(vals)
    assert np.array_equal(nvfp4.bf16_bits_to_f32(bits).astype(np.float64), vals)  # exact in bf16
    W = _rand_nvfp4(rng, N, K)
    off = np.array([0, R])
    assert np.array_equal(moe.grouped_gemm_w4a16(bits, off, lambda e: W, N, K),
                          moe.grouped_gemm(aq, sc, off, lambda e: W, N, K))


def test_w4a16_gemm_scales_exactly_with_the_activations():
    """Doubling every bf16 activation doubles every output exactly."""
    rng = np.random.default_rng(34)
    N, K = 5, 256
    a = _bf16_rows(rng, 2, K, -3, 3)
    a2 = (a.astype(np.int64) + (1 << 7)).astype(np.uint16)     # exponent + 1
    W = _rand_nvfp4(rng, N, K)
    off = np.array([0, 2])
    acc = moe.grouped_gemm_w4a16(a, off, lambda e: W, N, K)
    assert np.array_equal(moe.grouped_gemm_w4a16(a2, off, lambda e: W, N, K), 2 * acc)


def _run_w4a16(d, sel=None):
    T = d["x"].shape[0]
    idx = np.arange(len(d["a_expert"])) if sel is None else sel
    return moe.layer_forward_w4a16(d["x"], d["a_expert"][idx], d["a_src"][idx], d["a_dst"][idx],
                                   d["a_w"][idx], T, lambda e: d["W13"][e], lambda e: d["W2"][e],
                                   *d["g"], d["E"], d["H"], d["I"])


def test_w4a16_layer_single_row_closed_form():
    """One token routed to one expert with weight 0.5: out = bf16(0.5 * g_down * W2 @ h),
    h = bf16(silu(g_gate * Wg @ x) * g_up * Wu @ x), written out with exact rationals for
    the GEMMs and the logistic function in float64 (no oracle code)."""
    rng = np.random.default_rng(35)
    E, H, I = 2, 32, 16
    x = _bf16_rows(rng, 1, H)
    W13 = [_rand_nvfp4(rng, 2 * I, H, 0x28, 0x38) for _ in range(E)]
    W2 = [_rand_nvfp4(rng, H, I, 0x28, 0x38) for _ in range(E)]
    gg, gu, gd = (np.full(E, v, np.float32) for v in (0.75, 0.5, 0.25))
    out = moe.layer_forward_w4a16(x, np.array([1]), np.array([0]), np.array([0]),
                                  np.array([0.5], np.float32), 1, lambda e: W13[e],
                                  lambda e: W2[e], gg, gu, gd, E, H, I)
    xv = [_bf16_val(x[0, k]) for k in range(H)]
    zg = [float(0.75 * sum(xv[k] * _val(W13[1][0][j], W13[1][1][j], k) for k in range(H)))
          for j in range(I)]
    zu = [float(0.5 * sum(xv[k] * _val(W13[1][0][I + j], W13[1][1][I + j], k) for k in range(H)))
          for j in range(I)]
    h = nvfp4.f64_to_bf16_bits(np.array([g / (1.0 + np.exp(-g)) * u for g, u in zip(zg, zu)]))
    hv = [_bf16_val(b) if b & 0x7FFF else Fraction(0) for b in h]
    y = [float(Fraction(1, 8) * sum(hv[j] * _val(W2[1][0][n], W2[1][1][n], j) for j in range(I)))
         for n in range(H)]
    assert np.array_equal(out[0], nvfp4.f64_to_bf16_bits(np.array(y)))


def test_w4a16_layer_batch_parity_and_determinism():
    """[GG] "Proof" in W4A16 arithmetic: a token alone equals the token in its batch."""
    d = _tiny_layer_inputs(23)
    full = _run_w4a16(d)
    assert np.array_equal(_run_w4a16(d), full)
    k = d["k"]
    for t in (1, 4):
        alone = _run_w4a16(d, np.arange(t * k, t * k + k))
        assert np.array_equal(alone[t], full[t])


# --------------------------------------------------------------------------- W4A4 layer
def _w4a4_term_closed_form(x_row_bits, w13, w2, gg, gu, gd, rw, I, H):
    """One assignment's scatter term and its row globals, written out from the steps of
    [GG] "What changed" with the pinned quantizer, exact rational GEMMs and the logistic
    function in float64 (no other oracle code):
      xq, xs, gx = quantize(x);  ag[j], au[j] = exact sums of x_deq * w13_deq over k
      h = bf16( silu(gx * gg * ag) * (gx * gu * au) )       (per-half globals, option (a))
      hq, hs, gh = quantize(h);  y[n] = exact sum of h_deq * w2_deq over j
      term = rw * gd * gh * y                                (exact rational)"""
    xq, xs, gx = nvfp4.quantize_row(nvfp4.bf16_bits_to_f32(x_row_bits))
    xv = [_val(xq, xs, k) for k in range(H)]
    ag = [sum(xv[k] * _val(w13[0][j], w13[1][j], k) for k in range(H)) for j in range(I)]
    au = [sum(xv[k] * _val(w13[0][I + j], w13[1][I + j], k) for k in range(H))
          for j in range(I)]
    zg = [float(Fraction(float(gx)) * Fraction(float(gg)) * a) for a in ag]
    zu = [float(Fraction(float(gx)) * Fraction(float(gu)) * a) for a in au]
    h = nvfp4.f64_to_bf16_bits(np.array([g / (1.0 + np.exp(-g)) * u for g, u in zip(zg, zu)]))
    hq, hs, gh = nvfp4.quantize_row(nvfp4.bf16_bits_to_f32(h))
    hv = [_val(hq, hs, j) for j in range(I)]
    y = [sum(hv[j] * _val(w2[0][n], w2[1][n], j) for j in range(I)) for n in range(H)]
    c = Fraction(float(rw)) * Fraction(float(gd)) * Fraction(float(gh))
    return [c * v for v in y], float(gx), float(gh)


def _w4a4_case():
    """Three experts, two tokens: token 0 takes experts 2 and 0 (assignment order differs
    from the grouped order), token 1 expert 2 alone; gate, up and down globals differ."""
    rng = np.random.default_rng(36)
    E, H, I = 3, 32, 16
    x = _bf16_rows(rng, 2, H, -2, 2)
    # weight scales 2^-4 .. 2^-2: the SwiGLU inputs come out of order one, where silu is
    # far from both of its linear limits (a swapped pair of globals would cancel there)
    W13 = [_rand_nvfp4(rng, 2 * I, H, 0x18, 0x28) for _ in range(E)]
    W2 = [_rand_nvfp4(rng, H, I, 0x18, 0x28) for _ in range(E)]
    g = (np.array([0.5, 1.25, 0.75], np.float32), np.array([0.25, 1.5, 0.375], np.float32),
         np.array([0.125, 2.0, 0.5], np.float32))
    a = dict(a_expert=np.array([2, 0, 2]), a_src=np.array([0, 0, 1]),
             a_dst=np.array([0, 0, 1]), a_w=np.array([0.5, 0.25, 0.75], np.float32))
    return dict(x=x, W13=W13, W2=W2, g=g, E=E, H=H, I=I, T=2, **a)


def _w4a4_closed_form(d):
    T, H, I = d["T"], d["H"], d["I"]
    gg, gu, gd = d["g"]
    sums = [[Fraction(0)] * H for _ in range(T)]
    gxs, ghs = [], []
    for j in range(len(d["a_expert"])):
        e, s, t = int(d["a_expert"][j]), int(d["a_src"][j]), int(d["a_dst"][j])
        term, gx, gh = _w4a4_term_closed_form(d["x"][s], d["W13"][e], d["W2"][e], gg[e], gu[e],
                                              gd[e], d["a_w"][j], I, H)
        sums[t] = [a + b for a, b in zip(sums[t], term)]
        gxs.append(gx)
        ghs.append(gh)
    out = nvfp4.f64_to_bf16_bits(np.array([[float(v) for v in row] for row in sums]))
    return out, gxs, ghs


def _w4a4_oracle(d, sel=None):
    idx = np.arange(len(d["a_expert"])) if sel is None else np.asarray(sel)
    return moe.layer_forward(d["x"], d["a_expert"][idx], d["a_src"][idx], d["a_dst"][idx],
                             d["a_w"][idx], d["T"], lambda e: d["W13"][e], lambda e: d["W2"][e],
                             *d["g"], d["E"], d["H"], d["I"])


def test_w4a4_layer_single_row_closed_form():
    """[GG] "What changed": one token routed to one expert; the oracle's layer equals the
    closed form bit for bit, and the case separates the two row globals and the two
    halves' globals (so a swapped or dropped global would change the result)."""
    d = _w4a4_case()
    one = {**d, "a_expert": d["a_expert"][2:], "a_src": d["a_src"][2:],
           "a_dst": np.array([0]), "a_w": d["a_w"][2:], "T": 1}
    want, gxs, ghs = _w4a4_closed_form(one)
    assert gxs[0] != ghs[0] and gxs[0] != 1.0 and ghs[0] != 1.0
    got = _w4a4_oracle(one)
    assert np.array_equal(got, want)
    assert np.count_nonzero(got) > 0.9 * got.size


def test_w4a4_layer_multi_row_closed_form():
    """Two assignments of one token in the opposite of their grouped order, plus a second
    token: the oracle's grouping, router-weight permutation and per-token sum match the
    closed form (exact sum of the terms, rounded once to bf16)."""
    d = _w4a4_case()
    want, _, _ = _w4a4_closed_form(d)
    assert np.array_equal(_w4a4_oracle(d), want)


@pytest.mark.parametrize("mistake", ["swap_half_globals", "drop_x_global", "drop_h_global",
                                     "x_global_in_scatter", "weights_unpermuted"])
def test_w4a4_layer_closed_form_catches_wiring_mistakes(monkeypatch, mistake):
    """Plants each plausible wiring mistake in the oracle's layer (on the CPU) and checks
    that the closed-form pin above then fails: the pin constrains every global's place."""
    d = _w4a4_case()
    want, _, _ = _w4a4_closed_form(d)
    seen = {}
    swiglu, scatter, group = moe.swiglu, moe.scatter_add, moe.group_rows

    def bad_swiglu(acc13, offsets, g_gate, g_up, row_gs, I):
        seen["xgs"] = np.array(row_gs)
        if mistake == "swap_half_globals":
            g_gate, g_up = g_up, g_gate
        if mistake == "drop_x_global":
            row_gs = np.ones_like(row_gs)
        return swiglu(acc13, offsets, g_gate, g_up, row_gs, I)

    def bad_scatter(y, offsets, row_w, g_down, row_gs, tok_off, tok_rows, T):
        if mistake == "drop_h_global":
            row_gs = np.ones_like(row_gs)
        if mistake == "x_global_in_scatter":
            row_gs = seen["xgs"]
        return scatter(y, offsets, row_w, g_down, row_gs, tok_off, tok_rows, T)

    def bad_group(*args):
        g = group(*args)
        if mistake == "weights_unpermuted":
            g["row_w"] = np.asarray(args[3], np.float32).copy()
        return g

    monkeypatch.setattr(moe, "swiglu", bad_swiglu)
    monkeypatch.setattr(moe, "scatter_add", bad_scatter)
    monkeypatch.setattr(moe, "group_rows", bad_group)
    assert not np.array_equal(_w4a4_oracle(d), want)
