"""GPU parity of the W4A16 path (bf16 activations against NVFP4 weights) against the CPU
oracle, through the C ABI: grouped_gemm_w4a16 and moe_layer_forward_w4a16.

Bit-exact where every partial sum is exact (one-hot activations, small exact values);
otherwise GEMM max |gpu - oracle| <= 2e-3 x row RMS and the layer within 2% of the row RMS
on >= 99.9% of the elements, the bars of the W4A4 path.

[GG] is the page "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1
included, so the crossover is 1" (gabewillen.github.io/rocket).
"""
import numpy as np
import pytest

from oracle import moe as omoe
from oracle import nvfp4 as onv

from gpu_helpers import dev, empty, host, offsets_from_sizes, pack, rand_nvfp4, say, sync

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3
E2E_TOL = 0.02
E2E_FRAC = 0.999


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def run_w4a16(B, a_bits, offsets, wp, N, K):
    import torch
    R = a_bits.shape[0]
    E = len(offsets) - 1
    out = torch.full((max(R, 1), N), float("nan"), dtype=torch.float32, device="cuda")
    a = dev(a_bits) if R else empty((1, K), torch.int16)
    B.grouped_gemm_w4a16(a, dev(offsets), E, R, wp, N, K, out)
    sync()
    return host(out)[:R]


def _weights(B, rng, E, N, K, lo=0x20, hi=0x40):
    wn, wsc = rand_nvfp4(rng, E * N, K, lo, hi)
    return wn, wsc, pack(B, wn, wsc, E, N, K)


def _oracle(a_bits, offsets, wn, wsc, N, K):
    return omoe.grouped_gemm_w4a16(a_bits, offsets,
                                   lambda e: (wn[e * N:(e + 1) * N], wsc[e * N:(e + 1) * N]), N, K)


@pytest.mark.parametrize("K,N", [(2048, 512), (4096, 512), (640, 208), (1536, 208)])
def test_w4a16_gemm_random_within_tolerance(lib, K, N):
    """Random GEMMs within tolerance of the oracle; N = 208 leaves a partial item per
    expert and K = 640 / 1536 gives scale groups of 1 / 4 chunks."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("w4a16 gemm random K", K, "N", N)
    rng = np.random.default_rng(90 + K)
    sizes = [1, 3, 0, 4, 5, 7, 16, 18, 40, 2]
    E = len(sizes)
    off = offsets_from_sizes(sizes)
    R = int(off[-1])
    a = _bf16(rng.standard_normal((R, K)))
    wn, wsc, wp = _weights(B, rng, E, N, K)
    got = run_w4a16(B, a, off, wp, N, K)
    want = _oracle(a, off, wn, wsc, N, K)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    assert np.all(np.isfinite(got))
    err = np.abs(got - want)
    assert np.all(err <= GEMM_TOL * rms), float((err / rms).max())


def test_w4a16_gemm_exact_when_every_sum_is_exact(lib):
    """Activations +-1 / +-0.5 and weight scales 1.0: every product is a multiple of 1/4 up
    to 6, every partial sum of K = 256 fits in 13 bits, so fp32 accumulation is exact."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("w4a16 gemm exact")
    rng = np.random.default_rng(95)
    N, K = 64, 256
    sizes = [2, 0, 5, 17]
    E = len(sizes)
    off = offsets_from_sizes(sizes)
    R = int(off[-1])
    a = _bf16(rng.choice([-1.0, -0.5, 0.5, 1.0], size=(R, K)))
    wn = rng.integers(0, 256, (E * N, K // 2)).astype(np.uint8)
    wsc = np.full((E * N, K // 16), 0x38, np.uint8)
    wp = pack(B, wn, wsc, E, N, K)
    got = run_w4a16(B, a, off, wp, N, K)
    want = _oracle(a, off, wn, wsc, N, K)
    assert np.array_equal(got.astype(np.float64), want)


def test_w4a16_gemm_one_hot_activations_read_back_every_weight(lib):
    """x = 1.0 at one column per row: row i returns weight column k_i exactly, for columns
    spread over every chunk and both scale blocks of a lane."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("w4a16 gemm one-hot")
    rng = np.random.default_rng(96)
    N, K = 48, 1024
    cols = np.arange(0, K, 37)
    R = len(cols)
    a = np.zeros((R, K), np.uint16)
    a[np.arange(R), cols] = 0x3F80
    wn, wsc, wp = _weights(B, rng, 1, N, K, 0x00, 0x7E)
    off = np.array([0, R], np.int32)
    got = run_w4a16(B, a, off, wp, N, K)
    wd = onv.dequantize(wn, wsc)
    assert np.array_equal(got.astype(np.float64), wd[:, cols].T)


def test_w4a16_gemm_row_invariance_and_determinism(lib):
    """[GG] "Proof" in W4A16: a row alone equals the row grouped with others; repeated calls
    are bit-identical."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("w4a16 gemm invariance")
    rng = np.random.default_rng(97)
    N, K = 128, 2048
    a = _bf16(rng.standard_normal((33, K)))
    wn, wsc, wp = _weights(B, rng, 1, N, K)
    alone = np.concatenate([run_w4a16(B, a[i:i + 1], np.array([0, 1], np.int32), wp, N, K)
                            for i in range(33)])
    for g in (1, 5, 16, 17, 33):
        got = run_w4a16(B, a[:g], np.array([0, g], np.int32), wp, N, K)
        assert np.array_equal(got.view(np.uint32), alone[:g].view(np.uint32)), g
    again = [run_w4a16(B, a, np.array([0, 33], np.int32), wp, N, K) for _ in range(3)]
    for r in again[1:]:
        assert np.array_equal(r.view(np.uint32), again[0].view(np.uint32))


def test_w4a16_gemm_small_batch_instance_agrees_bitwise(lib):
    """A batch with no more rows than experts runs the small-batch instance (4 waves, 4 rows
    staged per pass: a group of 13 rows takes passes of 4, 4, 4 and 1 rows); the same rows
    in a larger batch run the 16-wave instance.  Both give the same bits (the instance
    changes which wave computes an output and how far ahead it loads, never the order of
    its accumulation), and both stay within tolerance of the oracle."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("w4a16 small-batch instance")
    rng = np.random.default_rng(98)
    E, N, K = 64, 256, 1024
    wn, wsc, wp = _weights(B, rng, E, N, K)
    big_sizes = np.full(E, 2)
    big_sizes[5], big_sizes[40] = 13, 1
    big_off = offsets_from_sizes(big_sizes)
    a = _bf16(rng.standard_normal((int(big_off[-1]), K)))
    big = run_w4a16(B, a, big_off, wp, N, K)            # 138 rows > 64 experts
    small_sizes = np.zeros(E, np.int64)
    small_sizes[5], small_sizes[40] = 13, 1
    rows = np.concatenate([np.arange(big_off[5], big_off[6]), np.arange(big_off[40], big_off[41])])
    small_off = offsets_from_sizes(small_sizes)
    small = run_w4a16(B, a[rows], small_off, wp, N, K)  # 14 rows <= 64 experts
    assert np.array_equal(small.view(np.uint32), big[rows].view(np.uint32))
    want = _oracle(a[rows], small_off, wn, wsc, N, K)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    assert np.all(np.abs(small - want) <= GEMM_TOL * rms)


def _out_f64(bits):
    return onv.bf16_bits_to_f32(np.asarray(bits).view(np.uint16)).astype(np.float64)


def _e2e_ok(got_bits, want_bits):
    got, want = _out_f64(got_bits), _out_f64(want_bits)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    ok = np.abs(got - want) <= E2E_TOL * rms
    return float(ok.mean()), float((np.abs(got - want) / np.maximum(rms, 1e-30)).max())


@pytest.mark.parametrize("name,shape", [("tiny", {}), ("ragged2303", dict(E=32, H=512, I=256)),
                                        ("zipf512", dict(E=48, H=256, I=384))])
def test_w4a16_layer_matches_oracle(lib, name, shape):
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("w4a16 layer", name, shape)
    wl = W.make_workload(name, **shape)
    dl = L.DeviceLayer(wl, arithmetic="w4a16")
    got = host(dl.forward()).view(np.uint16).copy()
    assert dl.device_error() == 0
    assert np.array_equal(host(dl.forward()).view(np.uint16), got)      # deterministic
    want = omoe.layer_forward_w4a16(wl.x, wl.a_expert, wl.a_src, wl.a_dst, wl.a_w, wl.T, wl.w13,
                                    wl.w2, wl.g_gate, wl.g_up, wl.g_down, wl.E, wl.H, wl.I)
    frac, worst = _e2e_ok(got, want)
    say("%s: fraction within tolerance %.5f, worst %.4f x RMS" % (name, frac, worst))
    assert frac >= E2E_FRAC


def test_w4a16_layer_batch_parity_and_graph_replay(lib):
    """A token alone equals the token in its batch; HIP-graph replays equal the eager call."""
    import torch
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("w4a16 batch parity / graph")
    wl = W.make_workload("zipf512", E=32, H=256, I=256)
    dl = L.DeviceLayer(wl, arithmetic="w4a16")
    full = host(dl.forward()).copy()
    g = dl.capture_graph()
    for _ in range(3):
        g.replay()
        sync()
        assert np.array_equal(host(dl.out), full)
        dl.forward()
        sync()
    for t in (0, 17, 63):
        sel = np.where(wl.a_dst == t)[0]
        one = W.Workload(**{**wl.__dict__, "a_expert": wl.a_expert[sel], "a_src": wl.a_src[sel],
                            "a_dst": wl.a_dst[sel], "a_w": wl.a_w[sel]})
        d1 = L.DeviceLayer(one, weights=(dl.w13, dl.w2), arithmetic="w4a16")
        alone = host(d1.forward())
        sync()
        assert np.array_equal(alone[t], full[t]), t
    del g
    torch.cuda.synchronize()


def test_w4a16_layer_eight_row_passes(lib):
    """A batch of at most 4 rows per expert on average and groups above 8 rows: the w13 GEMM
    runs 8-wave workgroups staging 8 rows per pass, so the large groups take several
    passes.  The layer stays within the end-to-end bar of the oracle, and a token computed
    alone (on the small-batch instances) has the same bits as in the batch."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("w4a16 eight-row passes")
    wl = W.make_workload("zipf512", E=160, H=256, I=256)
    assert wl.R <= 4 * wl.E and np.bincount(wl.a_expert, minlength=wl.E).max() > 8
    dl = L.DeviceLayer(wl, arithmetic="w4a16")
    full = host(dl.forward()).view(np.uint16).copy()
    assert dl.device_error() == 0
    want = omoe.layer_forward_w4a16(wl.x, wl.a_expert, wl.a_src, wl.a_dst, wl.a_w, wl.T, wl.w13,
                                    wl.w2, wl.g_gate, wl.g_up, wl.g_down, wl.E, wl.H, wl.I)
    frac, worst = _e2e_ok(full, want)
    say("fraction within tolerance %.5f, worst %.4f x RMS" % (frac, worst))
    assert frac >= E2E_FRAC
    hot = int(np.argmax(np.bincount(wl.a_expert, minlength=wl.E)))
    for t in sorted(set(wl.a_dst[wl.a_expert == hot].tolist()))[:2]:
        sel = np.where(wl.a_dst == t)[0]
        one = W.Workload(**{**wl.__dict__, "a_expert": wl.a_expert[sel], "a_src": wl.a_src[sel],
                            "a_dst": wl.a_dst[sel], "a_w": wl.a_w[sel]})
        d1 = L.DeviceLayer(one, weights=(dl.w13, dl.w2), arithmetic="w4a16")
        alone = host(d1.forward()).view(np.uint16)
        sync()
        assert np.array_equal(alone[t], full[t]), t


@pytest.mark.parametrize("R,T,H,I,hot", [(1, 1, 512, 256, 0), (8, 3, 512, 1024, 3),
                                         (12, 5, 1024, 2048, 5), (16, 1, 512, 512, 0),
                                         (16, 4, 1024, 256, 16), (8, 2, 512, 4096, 0)])
def test_w4a16_decode_layer_equals_the_batch_path(lib, R, T, H, I, hot):
    """Up to 16 assignments the W4A16 layer is two launches (the w2 launch also sums the
    tokens, at 8 or 16 waves per workgroup): every token's output equals the same token's
    output in a batch of more than 32 assignments (the general path: the w2 GEMM and the
    per-token sum as launches of their own) bit for bit, with a group of 3, 5 or 16 rows and
    one token of 16 rows."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("w4a16 decode layer vs batch path", R, T, H, I, hot)
    base = W.make_workload("ragged2303", E=24, H=H, I=I)
    rng = np.random.default_rng(1000 * R + T + I)
    a_expert = rng.choice(base.E, R, replace=False).astype(np.int32)
    a_expert[:hot] = 3
    a_src = rng.integers(0, base.S, R).astype(np.int32)
    a_dst = rng.integers(0, T, R).astype(np.int32)
    a_w = rng.uniform(0.05, 1.0, R).astype(np.float32)
    small = W.Workload(**{**base.__dict__, "T": T, "a_expert": a_expert, "a_src": a_src,
                          "a_dst": a_dst, "a_w": a_w})
    n = 40  # more assignments, to other tokens: the batch takes the general path
    big = W.Workload(**{**base.__dict__, "T": T + 10,
                        "a_expert": np.concatenate([a_expert, rng.integers(0, base.E, n)]).astype(np.int32),
                        "a_src": np.concatenate([a_src, rng.integers(0, base.S, n)]).astype(np.int32),
                        "a_dst": np.concatenate([a_dst, rng.integers(T, T + 10, n)]).astype(np.int32),
                        "a_w": np.concatenate([a_w, rng.uniform(0.05, 1.0, n)]).astype(np.float32)})
    d1 = L.DeviceLayer(small, arithmetic="w4a16")
    d2 = L.DeviceLayer(big, weights=(d1.w13, d1.w2), arithmetic="w4a16")
    got = host(d1.forward()).copy()
    want = host(d2.forward()).copy()
    sync()
    assert d1.device_error() == 0 and d2.device_error() == 0
    assert np.count_nonzero(got) > 0
    assert np.array_equal(got, want[:T])
