"""GPU parity of each library entry point against the CPU oracle, through the C ABI.

Bit-exact: weight packing, grouping / gather indices, quantized nibbles / scale bytes /
row globals, and GEMMs whose every partial sum is exact.  Tolerances elsewhere:
GEMM max |gpu - oracle| <= 2e-3 x row RMS (fp32 accumulation vs float64 over identical
exact operands); SwiGLU and scatter within one bf16 rounding step.

[GG] is the page "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1
included, so the crossover is 1"; [MF] the page "Fusing the MoE layer's two grouped GEMMs is
worth 4%, and a CUDA graph already collects it" (gabewillen.github.io/rocket).
"""
import numpy as np
import pytest

from oracle import moe as omoe
from oracle import nvfp4 as onv

from gpu_helpers import dev, empty, host, offsets_from_sizes, pack, rand_nvfp4, run_gemm, say, sync

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3


# ------------------------------------------------------------------------------ packing
def _sign_folded(nib, scl):
    """The canonical bytes nvfp4_unpack_weights documents for packed weights: every block
    scale with its sign bit cleared and, in those blocks, the e2m1 sign bits flipped."""
    neg = (scl & 0x80) != 0                                  # [rows, K/16]
    flip = np.repeat(neg, 8, axis=1).astype(np.uint8) * 0x88  # 8 bytes per 16-block
    return nib ^ flip, scl & 0x7F


def _values(nib, scl):
    v = onv.dequantize(nib, scl)
    return np.where(np.isnan(v), 1e30, v)  # NaN scales compare equal to each other


def test_pack_unpack_roundtrip_and_fused_concat(lib):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    rng = np.random.default_rng(1)
    for (E, N, K) in [(3, 48, 384), (2, 32, 4096), (1, 16, 128)]:
        for lo, hi in ((0, 0x7E), (0, 255)):
            say("pack", E, N, K, "scales", lo, hi)
            nib, scl = rand_nvfp4(rng, E * N, K, lo, hi)
            wp = pack(B, nib, scl, E, N, K)
            assert wp.numel() == E * N * K * 9 // 16
            nib2 = empty((E * N, K // 2), torch.uint8)
            scl2 = empty((E * N, K // 16), torch.uint8)
            B.nvfp4_unpack_weights(wp, E, N, K, nib2, scl2)
            sync()
            n2, s2 = host(nib2), host(scl2)
            fn, fs = _sign_folded(nib, scl)
            assert np.array_equal(n2, fn) and np.array_equal(s2, fs)
            if hi <= 0x7E:  # non-negative scales: an exact byte round trip
                assert np.array_equal(n2, nib) and np.array_equal(s2, scl)
            # the values (e2m1 x e4m3, signed zeros included) never change
            v0, v1 = _values(nib, scl), _values(n2, s2)
            assert np.array_equal(v0, v1) and np.array_equal(np.signbit(v0), np.signbit(v1))
    # fused gate|up packs to the concatenation of the separately packed halves
    I, K = 32, 256
    g, gs = rand_nvfp4(rng, I, K, 0, 255)
    u, us = rand_nvfp4(rng, I, K, 0, 255)
    fused = host(pack(B, np.concatenate([g, u]), np.concatenate([gs, us]), 1, 2 * I, K))
    sep = np.concatenate([host(pack(B, g, gs, 1, I, K)), host(pack(B, u, us, 1, I, K))])
    assert np.array_equal(fused, sep)


# ------------------------------------------------------------------------------ quantize
def _special_rows(K):
    rows = []
    rows.append(np.zeros(K, np.float32))
    x = np.zeros(K, np.float32)
    x[:16] = np.arange(1, 17)
    rows.append(x)
    x = np.zeros(K, np.float32)
    x[:16] = np.arange(-8, 8)
    rows.append(x)
    x = np.zeros(K, np.float32)
    x[:16] = [6, 3, 1.5, 0.75, 0.375, 0.1875, 0, -6, -3, -1.5, -0.75, -0.375, -0.1875, -0.0, 0.25, 2.5]
    rows.append(x)
    x = np.full(K, -0.0, np.float32)
    x[5] = 1.0
    rows.append(x)
    rng = np.random.default_rng(9)
    rows.append((rng.standard_normal(K) * 1e-39).astype(np.float32))    # bf16 subnormal range
    rows.append((rng.standard_normal(K) * 1e37).astype(np.float32))     # near the top
    x = (rng.standard_normal(K) * np.exp(rng.uniform(-12, 12, K))).astype(np.float32)
    rows.append(x)                                                     # blocks of every size
    x = rng.standard_normal(K).astype(np.float32)
    x[::16] = 0
    x[K // 2:K // 2 + 16] = 2.0 ** -30                                 # underflowing block scale
    rows.append(x)
    return np.stack(rows)


def _to_bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("K,R", [(64, 131), (16, 5), (256, 40), (2048, 24), (4096, 24), (8192, 4)])
def test_quantize_bit_exact(lib, K, R):
    """K=64 with 131 rows is the shape of the page's kernel check (groups of 1 and 130
    rows, [GG] "Proof")."""
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    say("quantize K=%d R=%d" % (K, R))
    rng = np.random.default_rng(K + R)
    x = (rng.standard_normal((R, K)) * np.exp(rng.uniform(-3, 3, (R, 1)))).astype(np.float32)
    if K >= 16:
        x = np.concatenate([x, _special_rows(K)])
    bits = _to_bf16_bits(x)
    R = bits.shape[0]
    q = empty((R, K // 2), torch.uint8)
    sc = empty((R, K // 16), torch.uint8)
    gs = empty((R,), torch.float32)
    B.nvfp4_quantize_rows(dev(bits), R, K, q, sc, gs)
    sync()
    wq, ws, wg = onv.quantize_rows(onv.bf16_bits_to_f32(bits))
    assert np.array_equal(host(q), wq)
    assert np.array_equal(host(sc), ws)
    assert np.array_equal(host(gs).view(np.uint32), wg.view(np.uint32))


def test_quantize_empty_batch(lib):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    B.nvfp4_quantize_rows(empty((1, 64), torch.int16), 0, 64, empty((1, 32), torch.uint8),
                          empty((1, 4), torch.uint8), empty((1,), torch.float32))
    sync()


# ------------------------------------------------------------------------------ group / gather
def _run_group(B, x, S, H, a_expert, a_src, a_dst, a_w, E, T):
    import torch
    R = len(a_expert)
    Rb = max(R, 1)
    outs = dict(xg=empty((Rb, H), torch.int16), offsets=empty((E + 1,), torch.int32),
                row_src=empty((Rb,), torch.int32), row_dst=empty((Rb,), torch.int32),
                row_w=empty((Rb,), torch.float32), tok_off=empty((T + 1,), torch.int32),
                tok_rows=empty((Rb,), torch.int32), err=empty((1,), torch.int32))
    B.moe_gather_rows(dev(x) if S else empty((1, H), torch.int16), S, H, dev(a_expert),
                      dev(a_src), dev(a_dst), dev(a_w), R, E, T, outs["xg"], outs["offsets"],
                      outs["row_src"], outs["row_dst"], outs["row_w"], outs["tok_off"],
                      outs["tok_rows"], outs["err"])
    err = B.moe_get_device_error(outs["err"])
    return {k: host(v) for k, v in outs.items()}, err


@pytest.mark.parametrize("case", ["random_invalid", "ragged570", "zipf", "empty", "one_expert",
                                  "many_experts", "ragged2303", "large_uncached", "max_experts",
                                  "small_invalid", "small_decode4", "small_one_row",
                                  "small_wide_keys", "small_one_expert", "small_33"])
def test_group_gather_bit_exact(lib, case):
    """Grouping and gather bit-exact against the oracle.  The "small_" cases have at most 32
    assignments (the one-wave grouping; "small_33" is the first size past it)."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("group", case)
    rng = np.random.default_rng(sum(map(ord, case)))
    H = 64
    if case == "random_invalid":
        E, S, T, R = 13, 20, 9, 300
        a_expert = rng.integers(-2, E + 2, R)
        a_src = rng.integers(-1, S + 1, R)
        a_dst = rng.integers(-1, T + 1, R)
    elif case == "ragged570":
        E, S, T, R = 288, 570, 8, 570
        a_expert = np.repeat(np.arange(E), 1 + rng.multinomial(R - E, np.full(E, 1 / E)))
        a_src = np.arange(R)
        a_dst = rng.integers(0, T, R)
    elif case == "zipf":
        E, S, T = 288, 64, 64
        p = (rng.permutation(E) + 1.0) ** -1.1
        a_expert = np.concatenate([rng.choice(E, 8, replace=False, p=p / p.sum()) for _ in range(T)])
        a_src = np.repeat(np.arange(T), 8)
        a_dst = a_src.copy()
        R = len(a_expert)
    elif case == "empty":
        E, S, T, R = 8, 4, 4, 0
        a_expert = a_src = a_dst = np.zeros(0, np.int64)
    elif case == "many_experts":      # key ranges too wide for per-wave histograms
        E, S, T, R = 3000, 700, 50, 700
        a_expert = rng.integers(-1, E + 1, R)
        a_src = np.arange(R)
        a_dst = rng.integers(0, T, R)
    elif case == "max_experts":       # E = 8192, the library's limit
        E, S, T, R = 8192, 512, 64, 512
        a_expert = rng.integers(0, E, R)
        a_src = np.arange(R)
        a_dst = rng.integers(0, T, R)
    elif case == "large_uncached":    # too many assignments to hold in LDS: global reads
        E, S, T, R = 64, 40000, 500, 40000
        a_expert = rng.integers(-1, E, R)
        a_src = np.arange(R)
        a_dst = rng.integers(0, T, R)
    elif case == "small_invalid":
        E, S, T, R = 13, 20, 9, 30
        a_expert = rng.integers(-2, E + 2, R)
        a_src = rng.integers(-1, S + 1, R)
        a_dst = rng.integers(-1, T + 1, R)
    elif case in ("small_decode4", "small_33"):   # top-8 of 288 for 4 tokens: R = 32
        E, T = 288, 4
        a_expert = np.concatenate([rng.choice(E, 8, replace=False) for _ in range(T)])
        a_src = np.repeat(np.arange(T), 8)
        a_dst = a_src.copy()
        if case == "small_33":
            a_expert, a_src, a_dst = (np.append(v, v[:1]) for v in (a_expert, a_src, a_dst))
        S, R = T, len(a_expert)
    elif case == "small_one_row":
        E, S, T, R = 288, 1, 1, 1
        a_expert, a_src, a_dst = np.array([287]), np.array([0]), np.array([0])
    elif case == "small_wide_keys":   # E and T far above 64: many offsets per lane
        E, S, T, R = 8192, 32, 5000, 32
        a_expert = rng.integers(-1, E, R)
        a_src = np.arange(R)
        a_dst = rng.integers(0, T, R)
    elif case == "small_one_expert":  # 32 equal keys: order by assignment index
        E, S, T, R = 6, 10, 3, 32
        a_expert = np.full(R, 5)
        a_src = rng.integers(0, S, R)
        a_dst = rng.integers(0, T, R)
    elif case == "ragged2303":
        E, S, T, R = 288, 2303, 288, 2303
        a_expert = np.repeat(np.arange(E), 1 + rng.multinomial(R - E, np.full(E, 1 / E)))
        a_src = np.arange(R)
        a_dst = rng.permutation(R) // 8
    else:
        E, S, T, R = 5, 3, 2, 100
        a_expert = np.full(R, 3)
        a_src = rng.integers(0, S, R)
        a_dst = rng.integers(0, T, R)
    a_w = rng.random(R).astype(np.float32)
    x = rng.integers(0, 65536, (max(S, 1), H)).astype(np.uint16)[:S]
    a_expert, a_src, a_dst = (np.asarray(v, np.int32) for v in (a_expert, a_src, a_dst))
    got, err = _run_group(B, x, S, H, a_expert, a_src, a_dst, a_w, E, T)
    want = omoe.group_rows(a_expert, a_src, a_dst, a_w, E, S, T)
    assert err == want["err"]
    assert np.array_equal(got["offsets"], want["offsets"])
    assert np.array_equal(got["tok_off"], want["tok_off"])
    if R:
        assert np.array_equal(got["row_src"][:R], want["row_src"])
        assert np.array_equal(got["row_dst"][:R], want["row_dst"])
        assert np.array_equal(got["row_w"][:R].view(np.uint32), want["row_w"].view(np.uint32))
        Rv = int(want["offsets"][E])
        assert np.array_equal(got["tok_rows"][:Rv], want["tok_rows"])
        xg = omoe.gather_rows(x, want["row_src"])
        assert np.array_equal(got["xg"][:R].view(np.uint16), xg)


# ------------------------------------------------------------------------------ GEMM
def _oracle_gemm(aq, as_, offsets, wnib, wscl, E, N, K):
    return omoe.grouped_gemm(aq, as_, offsets,
                             lambda e: (wnib[e * N:(e + 1) * N], wscl[e * N:(e + 1) * N]), N, K)


SIZES = [1, 2, 0, 3, 4, 5, 16, 17, 33, 8, 0, 1]


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_gemm_exact_arithmetic_bit_exact(lib, flags):
    """All scales 1.0: every product is a multiple of 1/4 and every partial sum over
    K = 4096 is exact in fp32, so any summation order gives the oracle's value exactly."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm exact flags", flags)
    rng = np.random.default_rng(20 + flags)
    N, K = 256, 4096
    E = len(SIZES)
    offsets = offsets_from_sizes(SIZES)
    R = int(offsets[-1])
    aq, as_ = rand_nvfp4(rng, R, K, 0x38, 0x38)
    wn, ws = rand_nvfp4(rng, E * N, K, 0x38, 0x38)
    wp = pack(B, wn, ws, E, N, K)
    got = run_gemm(B, aq, as_, offsets, wp, N, K, flags)
    want = _oracle_gemm(aq, as_, offsets, wn, ws, E, N, K)
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("flags", [1, 2])
def test_gemm_one_hot_activations_read_back_every_weight(lib, flags):
    """One-hot activation rows (a single 1.0) turn the GEMM into a read-back of the
    dequantized weights: exact for every e2m1 code times every finite e4m3 scale code."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm one-hot activations flags", flags)
    rng = np.random.default_rng(30 + flags)
    N, K = 64, 256
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2                  # 1.0
    aq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    as_ = np.full((K, K // 16), 0x38, np.uint8)
    wn = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    ws = finite[rng.integers(0, len(finite), (N, K // 16))]
    ws[:16, :] = np.resize(finite, 16 * (K // 16)).reshape(16, K // 16)  # every code appears
    wp = pack(B, wn, ws, 1, N, K)
    offsets = np.array([0, K], np.int32)
    got = run_gemm(B, aq, as_, offsets, wp, N, K, flags)
    want = onv.dequantize(wn, ws).T                        # [K, N]
    assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("flags", [1, 2])
def test_gemm_one_hot_weights_read_back_every_activation(lib, flags):
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm one-hot weights flags", flags)
    rng = np.random.default_rng(40 + flags)
    N = K = 128
    perm = rng.permutation(K)
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), perm] = 2
    wn = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ws = np.full((N, K // 16), 0x38, np.uint8)
    wp = pack(B, wn, ws, 1, N, K)
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    R = 21
    aq = rng.integers(0, 256, (R, K // 2)).astype(np.uint8)
    as_ = finite[rng.integers(0, len(finite), (R, K // 16))]
    got = run_gemm(B, aq, as_, np.array([0, R], np.int32), wp, N, K, flags)
    want = onv.dequantize(aq, as_)[:, perm]
    assert np.array_equal(got.astype(np.float64), want)


def _workload_like(rng, R, K):
    """Activation rows quantized by the oracle from bf16 N(0,1); weights as in the bench."""
    x = _to_bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    aq, as_, _ = onv.quantize_rows(onv.bf16_bits_to_f32(x))
    return aq, as_


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_gemm_random_within_tolerance(lib, flags):
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("gemm random flags", flags)
    rng = np.random.default_rng(50 + flags)
    N, K = 512, 4096
    sizes = [1, 3, 0, 4, 5, 7, 16, 18, 40, 2]
    E = len(sizes)
    offsets = offsets_from_sizes(sizes)
    R = int(offsets[-1])
    aq, as_ = _workload_like(rng, R, K)
    ws_ = [W.expert_weights(77, e, 0, N, K) for e in range(E)]
    wn = np.concatenate([w[0] for w in ws_])
    wsc = np.concatenate([w[1] for w in ws_])
    wp = pack(B, wn, wsc, E, N, K)
    got = run_gemm(B, aq, as_, offsets, wp, N, K, flags)
    want = _oracle_gemm(aq, as_, offsets, wn, wsc, E, N, K)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    assert np.all(err <= GEMM_TOL * rms), float((err / rms).max())


@pytest.mark.parametrize("flags", [1, 2])
@pytest.mark.parametrize("K", [384, 640, 1152, 1536])
def test_gemm_ragged_tiles_and_odd_scale_groups(lib, flags, K):
    """N = 208 (13 tiles: one whole 8-tile item and a partial one per expert) and K with
    3, 5, 9 or 12 chunks (scale groups of 1, 1, 1 and 4 chunks, rings of 1 to 4): random
    GEMMs within tolerance of the oracle, and a row alone equals the row in its group."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("gemm ragged tiles K", K, "flags", flags)
    rng = np.random.default_rng(K + flags)
    N = 208
    sizes = [1, 7, 0, 20]
    E = len(sizes)
    offsets = offsets_from_sizes(sizes)
    R = int(offsets[-1])
    aq, as_ = _workload_like(rng, R, K)
    ws_ = [W.expert_weights(91, e, 0, N, K) for e in range(E)]
    wn = np.concatenate([w[0] for w in ws_])
    wsc = np.concatenate([w[1] for w in ws_])
    wp = pack(B, wn, wsc, E, N, K)
    got = run_gemm(B, aq, as_, offsets, wp, N, K, flags)
    want = _oracle_gemm(aq, as_, offsets, wn, wsc, E, N, K)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - want) <= GEMM_TOL * rms), float((np.abs(got - want) / rms).max())
    r = int(offsets[3]) + 13                       # a row of the 20-row group, alone
    alone_off = offsets_from_sizes([0, 0, 0, 1])
    alone = run_gemm(B, aq[r:r + 1], as_[r:r + 1], alone_off, wp, N, K, flags)
    assert np.array_equal(alone.view(np.uint32), got[r:r + 1].view(np.uint32))


@pytest.mark.parametrize("flags", [0, 2])
def test_gemm_largest_k_smallest_n(lib, flags):
    """K = 8192 (64 chunks, eight scale groups) with N = 16 (a single tile per expert)."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm K=8192 N=16", flags)
    rng = np.random.default_rng(110 + flags)
    N, K = 16, 8192
    sizes = [3, 0, 17]
    E = len(sizes)
    off = offsets_from_sizes(sizes)
    aq, as_ = _workload_like(rng, int(off[-1]), K)
    wn, wsc = rand_nvfp4(rng, E * N, K, 0x20, 0x40)
    wp = pack(B, wn, wsc, E, N, K)
    got = run_gemm(B, aq, as_, off, wp, N, K, flags, gemv_max=0)
    want = _oracle_gemm(aq, as_, off, wn, wsc, E, N, K)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    err = np.abs(got - want)
    assert np.all(err <= GEMM_TOL * rms), float((err / rms).max())


@pytest.mark.parametrize("flags,sizes", [(1, [1, 2, 3, 4]), (2, [1, 5, 8, 16, 17, 33])])
def test_gemm_row_invariance_within_path(lib, flags, sizes):
    """[GG] "Proof": a row's output is the same alone or grouped."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm row invariance", flags, sizes)
    rng = np.random.default_rng(60 + flags)
    N, K = 128, 2048
    aq, as_ = _workload_like(rng, max(sizes), K)
    wn, wsc = rand_nvfp4(rng, N, K, 0x20, 0x40)
    wp = pack(B, wn, wsc, 1, N, K)
    alone = np.concatenate([run_gemm(B, aq[i:i + 1], as_[i:i + 1], np.array([0, 1], np.int32), wp,
                                     N, K, flags) for i in range(max(sizes))])
    for g in sizes:
        grouped = run_gemm(B, aq[:g], as_[:g], np.array([0, g], np.int32), wp, N, K, flags)
        assert np.array_equal(grouped.view(np.uint32), alone[:g].view(np.uint32)), g


@pytest.mark.parametrize("K", [2048, 4096])
def test_gemm_double_passes_equal_single_rows_and_oracle(lib, K):
    """Groups of more than 16 rows at a K with an even number of scale groups take double
    passes (up to 32 rows against one stream of the weights, staged over half of K at a
    time), the rest of a group single passes: every output within the GEMM tolerance of the
    oracle, and the rows at each pass boundary equal to the same rows computed alone, bit
    for bit ([GG] "Proof": a row's output does not depend on its group)."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm double passes", K)
    rng = np.random.default_rng(130 + K // 1024)
    N = 256
    sizes = [17, 25, 32, 33, 40, 57, 64, 65, 3]
    E = len(sizes)
    off = offsets_from_sizes(sizes)
    aq, as_ = _workload_like(rng, int(off[-1]), K)
    wn, wsc = rand_nvfp4(rng, E * N, K, 0x20, 0x40)
    wp = pack(B, wn, wsc, E, N, K)
    got = run_gemm(B, aq, as_, off, wp, N, K, 2, gemv_max=0)
    want = _oracle_gemm(aq, as_, off, wn, wsc, E, N, K)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    assert np.all(np.abs(got - want) <= GEMM_TOL * rms), float((np.abs(got - want) / rms).max())
    for e, g in enumerate(sizes):
        for k in sorted({0, 15, 16, 31, 32, 47, 48, 63, 64, g - 1}):
            if k >= g:
                continue
            r = int(off[e]) + k
            alone = run_gemm(B, aq[r:r + 1], as_[r:r + 1],
                             offsets_from_sizes([0] * e + [1] + [0] * (E - e - 1)), wp, N, K, 2,
                             gemv_max=0)
            assert np.array_equal(alone.view(np.uint32), got[r:r + 1].view(np.uint32)), (e, k)


@pytest.mark.parametrize("flags", [0, 2])
def test_gemm_grid_paths_agree_bitwise(lib, flags):
    """A small batch (few non-empty groups: the deep-ring, one-tile-per-wave instance) and a
    large one (the two-tiles-per-wave instance) give the same bits for the same rows: the
    instance changes which wave computes an output, never its accumulation order."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm grid paths", flags)
    rng = np.random.default_rng(80 + flags)
    E, N, K = 600, 1024, 256
    wn, wsc = rand_nvfp4(rng, E * N, K, 0x20, 0x40)
    wp = pack(B, wn, wsc, E, N, K)
    sizes = np.full(E, 2)
    big_off = offsets_from_sizes(sizes)
    aq, as_ = _workload_like(rng, int(big_off[-1]), K)
    big = run_gemm(B, aq, as_, big_off, wp, N, K, flags, gemv_max=0)  # 600 groups: large grid
    pick = [0, 299, 599]
    rows = np.concatenate([np.arange(big_off[e], big_off[e + 1]) for e in pick])
    small_sizes = np.zeros(E, np.int64)
    small_sizes[pick] = 2
    small_off = offsets_from_sizes(small_sizes)
    small = run_gemm(B, aq[rows], as_[rows], small_off, wp, N, K, flags, gemv_max=0)  # 3 groups
    assert np.array_equal(small.view(np.uint32), big[rows].view(np.uint32))


@pytest.mark.parametrize("flags", [1, 2])
def test_gemm_fused_w13_equals_separate_and_is_deterministic(lib, flags):
    """[GG] "Proof": fused gate|up == gate-only and up-only GEMMs,
    and five repeated calls are bit-identical."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("gemm fused/determinism", flags)
    rng = np.random.default_rng(70 + flags)
    I, K = 256, 1024
    sizes = [3, 6, 20]
    offsets = offsets_from_sizes(sizes)
    R = int(offsets[-1])
    E = len(sizes)
    aq, as_ = _workload_like(rng, R, K)
    gate = [rand_nvfp4(rng, I, K, 0x20, 0x40) for _ in range(E)]
    up = [rand_nvfp4(rng, I, K, 0x20, 0x40) for _ in range(E)]
    fn = np.concatenate([np.concatenate([g[0], u[0]]) for g, u in zip(gate, up)])
    fs = np.concatenate([np.concatenate([g[1], u[1]]) for g, u in zip(gate, up)])
    fused = run_gemm(B, aq, as_, offsets, pack(B, fn, fs, E, 2 * I, K), 2 * I, K, flags)
    g_only = run_gemm(B, aq, as_, offsets, pack(B, np.concatenate([g[0] for g in gate]),
                                                 np.concatenate([g[1] for g in gate]), E, I, K),
                      I, K, flags)
    u_only = run_gemm(B, aq, as_, offsets, pack(B, np.concatenate([u[0] for u in up]),
                                                 np.concatenate([u[1] for u in up]), E, I, K),
                      I, K, flags)
    assert np.array_equal(fused[:, :I].view(np.uint32), g_only.view(np.uint32))
    assert np.array_equal(fused[:, I:].view(np.uint32), u_only.view(np.uint32))
    wp = pack(B, fn, fs, E, 2 * I, K)
    for _ in range(5):
        again = run_gemm(B, aq, as_, offsets, wp, 2 * I, K, flags)
        assert np.array_equal(again.view(np.uint32), fused.view(np.uint32))


# ------------------------------------------------------------------------------ SwiGLU
def test_swiglu_within_one_bf16_step(lib):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    say("swiglu")
    rng = np.random.default_rng(80)
    I, E = 2048, 6
    sizes = [3, 0, 5, 1, 0, 7]
    offsets = offsets_from_sizes(sizes)
    R = int(offsets[-1]) + 2                      # two rows outside every group
    acc = (rng.standard_normal((R, 2 * I)) * 40000).astype(np.float32)
    gs = (rng.uniform(0.5, 2, R) * 1e-3).astype(np.float32)
    g_gate = (rng.uniform(0.5, 2, E) * 4.65e-2).astype(np.float32)
    g_up = (rng.uniform(0.5, 2, E) * 3.78e-2).astype(np.float32)
    h = empty((R, I), torch.int16)
    B.swiglu_grouped(dev(acc), R, I, dev(offsets), E, dev(g_gate), dev(g_up), dev(gs), h)
    sync()
    got = onv.bf16_bits_to_f32(host(h).view(np.uint16)).astype(np.float64)
    want = onv.bf16_bits_to_f32(omoe.swiglu(acc.astype(np.float64), offsets, g_gate, g_up, gs, I))
    want = want.astype(np.float64)
    ulp = np.abs(want) * 2.0 ** -7 + 1e-38
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == want) > 0.98
    assert not got[offsets[-1]:].any()


# ------------------------------------------------------------------------------ scatter
def test_scatter_within_bf16_rounding(lib):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    say("scatter")
    rng = np.random.default_rng(90)
    E, H, T = 7, 4096, 9
    sizes = [4, 0, 9, 2, 30, 1, 3]
    offsets = offsets_from_sizes(sizes)
    R = int(offsets[-1])
    a_dst = rng.integers(0, T - 1, R).astype(np.int32)     # token T-1 gets no rows
    a_expert = np.repeat(np.arange(E), sizes).astype(np.int32)
    g = omoe.group_rows(a_expert, np.zeros(R, np.int32), a_dst, np.ones(R, np.float32), E, 1, T)
    y = (rng.standard_normal((R, H)) * 1e5).astype(np.float32)
    row_w = rng.random(R).astype(np.float32)
    g_down = (rng.uniform(0.5, 2, E) * 4.2e-5).astype(np.float32)
    gs = (rng.uniform(0.5, 2, R) * 1e-8).astype(np.float32)
    out = empty((T, H), torch.int16)
    B.moe_scatter_add(dev(y), R, H, dev(offsets), E, dev(row_w), dev(g_down), dev(gs),
                      dev(g["tok_off"]), dev(g["tok_rows"]), T, out)
    sync()
    got = onv.bf16_bits_to_f32(host(out).view(np.uint16)).astype(np.float64)
    want = onv.bf16_bits_to_f32(omoe.scatter_add(y.astype(np.float64), offsets, row_w, g_down, gs,
                                                 g["tok_off"], g["tok_rows"], T)).astype(np.float64)
    scale = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True)) + 1e-30
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-5 * scale)
    assert not got[T - 1].any()


# ------------------------------------------------------------------------------ read probe
@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
def test_read_probe_reads_every_byte_it_is_given(lib, variant):
    """moe_hbm_read_probe (the measured read roofline) reads the whole buffer: one 16-byte
    word planted at the first, a middle and the last position is seen (the sink takes the
    key only when some lane's XOR fold equals it), and nothing is written otherwise."""
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    unit = 294912
    nbytes = 2 * unit
    key = 0x12345678
    for off in (0, nbytes // 2 + 1024 * 5 + 48, nbytes - 16):
        say("read probe variant", variant, "offset", off)
        buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        word = torch.tensor([key, 0, 0, 0], dtype=torch.int64).to(torch.int32)
        buf[off:off + 16] = word.view(torch.uint8).cuda()
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.moe_hbm_read_probe(buf, nbytes, variant, key + 1, sink)
        sync()
        assert int(sink.item()) == 0
        B.moe_hbm_read_probe(buf, nbytes, variant, key, sink)
        sync()
        assert int(sink.item()) == key
