"""End-to-end layer parity on the GPU, through moe_layer_forward.

Tolerance (end to end): |gpu - oracle| <= 2% of the oracle row's RMS on >= 99.9% of the
elements.  The two re-quantizations can flip a code where the GPU's fp32 and the oracle's
float64 SwiGLU output round to different bf16 neighbours, so exact equality is not the
bar here; it is for the layer against the same steps called one by one on the GPU.

[GG] is the page "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1
included, so the crossover is 1"; [MF] the page "Fusing the MoE layer's two grouped GEMMs is
worth 4%, and a CUDA graph already collects it" (gabewillen.github.io/rocket).
"""
import numpy as np
import pytest

from oracle import moe as omoe
from oracle import nvfp4 as onv

from gpu_helpers import composed_layer, dev, empty, host, say, sync

pytestmark = pytest.mark.gpu

E2E_TOL = 0.02
E2E_FRAC = 0.999


def _out_f64(bits):
    return onv.bf16_bits_to_f32(np.asarray(bits).view(np.uint16)).astype(np.float64)


def _e2e_ok(got_bits, want_bits):
    got, want = _out_f64(got_bits), _out_f64(want_bits)
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    ok = np.abs(got - want) <= E2E_TOL * rms
    return float(ok.mean()), float((np.abs(got - want) / np.maximum(rms, 1e-30)).max())


def _oracle_tokens(wl, tokens):
    """Oracle output rows of the given tokens (each token only needs its own rows)."""
    sel = np.where(np.isin(wl.a_dst, tokens))[0]
    out = omoe.layer_forward(wl.x, wl.a_expert[sel], wl.a_src[sel], wl.a_dst[sel], wl.a_w[sel],
                             wl.T, wl.w13, wl.w2, wl.g_gate, wl.g_up, wl.g_down, wl.E, wl.H, wl.I)
    return out[tokens]


# ------------------------------------------------------------------------------ tiny
@pytest.fixture(scope="module")
def tiny():
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload("tiny")
    return wl, L.DeviceLayer(wl)


def test_tiny_layer_matches_oracle(lib, tiny):
    wl, dl = tiny
    say("layer tiny")
    got = host(dl.forward()).view(np.uint16)
    sync()
    assert dl.device_error() == 0
    want = omoe.layer_forward(wl.x, wl.a_expert, wl.a_src, wl.a_dst, wl.a_w, wl.T, wl.w13, wl.w2,
                              wl.g_gate, wl.g_up, wl.g_down, wl.E, wl.H, wl.I)
    frac, worst = _e2e_ok(got, want)
    say("tiny: fraction within tolerance %.5f, worst %.4f x RMS" % (frac, worst))
    assert frac >= E2E_FRAC


@pytest.mark.parametrize("flags,gemv_max", [(0, 4), (1, 4), (2, 4), (0, 0)])
def test_layer_equals_separate_calls(lib, flags, gemv_max):
    """The fused layer (gather inside quantize, quantize inside SwiGLU) is bit-identical
    to the seven entry points called one after the other."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("layer vs separate calls", flags, gemv_max)
    wl = W.make_workload("ragged2303", E=24, H=512, I=256)
    dl = L.DeviceLayer(wl, flags=flags, gemv_max_rows=gemv_max)
    got = host(dl.forward())
    sync()
    assert np.array_equal(got, composed_layer(B, dl, flags, gemv_max))


@pytest.mark.parametrize("name,E,H,I", [("zipf512", 24, 1536, 768), ("zipf512", 40, 1024, 512),
                                        ("ragged2303", 16, 4096, 2048)])
def test_layer_multi_pass_groups_equal_separate_calls(lib, name, E, H, I):
    """Groups of 17 to ~170 rows (two to eleven 16-row passes over the same weights, the
    passes of an item in one workgroup, multi-pass groups first in the work list) at 12, 8
    and 32 items per expert: the layer is bit-identical to the separate entry points, which
    find their groups by scanning the offsets."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("multi-pass groups vs separate calls", name, E, H, I)
    wl = W.make_workload(name, E=E, H=H, I=I)
    sizes = np.bincount(wl.a_expert, minlength=E)
    assert (sizes > 16).any()
    dl = L.DeviceLayer(wl, flags=0, gemv_max_rows=0)
    got = host(dl.forward())
    sync()
    assert dl.device_error() == 0
    assert np.array_equal(got, composed_layer(B, dl, 0, 0))


@pytest.mark.parametrize("R,hot", [(1, 0), (17, 17), (32, 20), (33, 20)])
def test_decode_sized_layer_equals_separate_calls(lib, R, hot):
    """Batches of at most 32 assignments take the w13 launch that groups and quantizes by
    itself (no grouping launch): bit-identical to the separate entry points, with a group
    of more than 16 rows (two passes), two invalid assignments (dropped, error bits set) and
    33 assignments (the other path) as edge cases."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("decode-sized layer vs separate calls", R, hot)
    base = W.make_workload("ragged2303", E=24, H=512, I=256)
    sel = np.arange(R)
    a_expert = base.a_expert[sel].copy()
    a_expert[:hot] = 3  # one group of `hot` rows
    a_dst = base.a_dst[sel].copy()
    if R >= 17:
        a_expert[5] = base.E      # expert id out of range
        a_dst[6] = base.T         # output row out of range
    wl = W.Workload(**{**base.__dict__, "a_expert": a_expert, "a_src": base.a_src[sel],
                       "a_dst": a_dst, "a_w": base.a_w[sel]})
    dl = L.DeviceLayer(wl, flags=0, gemv_max_rows=0)
    got = host(dl.forward())
    sync()
    err = dl.device_error()
    assert err == (0 if R < 17 else B.MOE_ERR_EXPERT | B.MOE_ERR_DST), err
    assert np.array_equal(got, composed_layer(B, dl, 0, 0))


@pytest.mark.parametrize("R,hot", [(1, 0), (8, 0), (20, 18)])
def test_single_source_row_layer_equals_separate_calls(lib, R, hot):
    """One source row (a single decode token): the decode-sized w13 launch takes the
    instance that loads the row's blocks before it groups; bit-identical to the separate
    entry points, with one group of 18 rows of that row (two passes: the first from the
    loaded blocks, the second loading them again) and two dropped assignments."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("single-source-row layer vs separate calls", R, hot)
    base = W.make_workload("ragged2303", E=24, H=512, I=256)
    a_expert = (np.arange(R) % base.E).astype(np.int32)
    a_expert[:hot] = 5
    a_src = np.zeros(R, np.int32)
    a_dst = np.zeros(R, np.int32)
    if R >= 8:
        a_expert[3] = base.E    # expert id out of range
        a_src[4] = 1            # source row out of range
    a_w = np.linspace(0.1, 1.0, R).astype(np.float32)
    wl = W.Workload(**{**base.__dict__, "x": base.x[:1], "S": 1, "T": 1, "a_expert": a_expert,
                       "a_src": a_src, "a_dst": a_dst, "a_w": a_w})
    dl = L.DeviceLayer(wl, flags=0, gemv_max_rows=0)
    got = host(dl.forward())
    sync()
    err = dl.device_error()
    assert err == (0 if R < 8 else B.MOE_ERR_EXPERT | B.MOE_ERR_SRC), err
    assert np.array_equal(got, composed_layer(B, dl, 0, 0))


@pytest.mark.parametrize("R,T,I,hot,bad", [(8, 3, 1024, 3, False), (8, 100, 4096, 0, True),
                                            (12, 80, 256, 5, True), (16, 1, 2048, 0, False),
                                            (16, 4, 512, 16, False), (9, 9, 2048, 0, False),
                                            (8, 5, 2048, 2, True), (1, 1, 2048, 0, False)])
def test_w2_and_token_sum_launch_equals_separate_calls(lib, R, T, I, hot, bad):
    """Up to 16 assignments the w2 launch also sums each token's terms (the layer is two
    launches): bit-identical to the separate entry points at 8 and 16 waves per workgroup,
    K = 256 to 4096, a group of 3, 5 or 16 rows, one token of 16 rows (the per-token sum's
    eight partials of two rows each), more than 64 tokens (token offsets past the ones the
    launch caches), tokens without rows and dropped assignments."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("w2 + token-sum launch vs separate calls", R, T, I, hot, bad)
    base = W.make_workload("ragged2303", E=24, H=512, I=I)
    rng = np.random.default_rng(1000 * R + T)
    a_expert = rng.choice(base.E, R, replace=False).astype(np.int32)
    a_expert[:hot] = 3
    a_src = rng.integers(0, base.S, R).astype(np.int32)
    a_dst = rng.integers(0, T, R).astype(np.int32)
    if T > 64:
        a_dst[:4] = [0, 64, 65, T - 1]
    if bad:
        a_expert[R - 1] = base.E  # expert id out of range
        a_dst[R - 2] = T          # output row out of range
    a_w = rng.uniform(0.05, 1.0, R).astype(np.float32)
    wl = W.Workload(**{**base.__dict__, "T": T, "a_expert": a_expert, "a_src": a_src,
                       "a_dst": a_dst, "a_w": a_w})
    dl = L.DeviceLayer(wl, flags=0, gemv_max_rows=0)
    got = host(dl.forward())
    sync()
    err = dl.device_error()
    assert err == (B.MOE_ERR_EXPERT | B.MOE_ERR_DST if bad else 0), err
    assert np.array_equal(got, composed_layer(B, dl, 0, 0))
    assert np.count_nonzero(got) > 0


@pytest.mark.parametrize("flags", [1, 2])
def test_layer_batch_parity_and_determinism(lib, flags):
    """[GG] "Proof" / batch parity: a token's output is the same
    computed alone or inside the batch (within one GEMM path), and repeated calls are
    bit-identical."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("batch parity", flags)
    wl = W.make_workload("zipf512", E=32, H=256, I=256)
    dl = L.DeviceLayer(wl, flags=flags)
    full = host(dl.forward()).copy()
    for _ in range(4):
        assert np.array_equal(host(dl.forward()), full)
    for t in (0, 17, 63):
        sel = np.where(wl.a_dst == t)[0]
        one = W.Workload(**{**wl.__dict__, "a_expert": wl.a_expert[sel], "a_src": wl.a_src[sel],
                            "a_dst": wl.a_dst[sel], "a_w": wl.a_w[sel]})
        d1 = L.DeviceLayer(one, flags=flags, weights=(dl.w13, dl.w2))
        alone = host(d1.forward())
        sync()
        assert np.array_equal(alone[t], full[t]), t
        assert not np.delete(alone, t, axis=0).any()


def test_layer_batch_parity_across_grid_paths(lib):
    """Batch parity where the full batch runs the large-grid GEMM instances (w13 with the
    SwiGLU epilogue and w2, both above the small-grid threshold) and a single token the
    small-grid ones: the token's output bits are the same."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("batch parity across grid paths")
    wl = W.make_workload("zipf512", E=160, H=2048, I=1024)
    dl = L.DeviceLayer(wl)
    full = host(dl.forward()).copy()
    assert dl.device_error() == 0
    for t in (3, 40):
        sel = np.where(wl.a_dst == t)[0]
        one = W.Workload(**{**wl.__dict__, "a_expert": wl.a_expert[sel], "a_src": wl.a_src[sel],
                            "a_dst": wl.a_dst[sel], "a_w": wl.a_w[sel]})
        d1 = L.DeviceLayer(one, weights=(dl.w13, dl.w2))
        alone = host(d1.forward())
        sync()
        assert np.array_equal(alone[t], full[t]), t


def test_layer_drops_invalid_assignments(lib):
    """Out-of-range expert / source / output ids set the device error word and are
    dropped; the rest of the batch is computed as if they were absent."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    from nvfp4_block_scaled_gather_amd import binding as B
    say("invalid assignments")
    wl = W.make_workload("tiny")
    clean = L.DeviceLayer(wl)
    want = host(clean.forward()).copy()
    bad = W.Workload(**{**wl.__dict__,
                        "a_expert": np.concatenate([wl.a_expert, [wl.E, 1, 2]]).astype(np.int32),
                        "a_src": np.concatenate([wl.a_src, [0, wl.S + 3, 1]]).astype(np.int32),
                        "a_dst": np.concatenate([wl.a_dst, [1, 0, -1]]).astype(np.int32),
                        "a_w": np.concatenate([wl.a_w, [1, 1, 1]]).astype(np.float32)})
    dl = L.DeviceLayer(bad, weights=(clean.w13, clean.w2))
    got = host(dl.forward())
    assert dl.device_error() == B.MOE_ERR_EXPERT | B.MOE_ERR_SRC | B.MOE_ERR_DST
    assert np.array_equal(got, want)
    assert clean.device_error() == 0


@pytest.mark.parametrize("arithmetic", ["w4a4", "w4a16"])
def test_layer_empty_batch_and_tokens_without_rows(lib, arithmetic):
    """No assignments at all: every output row is zero and no error is raised.  Tokens
    that no assignment routes to come out zero while the others are unchanged."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("empty batch / idle tokens", arithmetic)
    wl = W.make_workload("tiny")
    base = L.DeviceLayer(wl, arithmetic=arithmetic)
    want = host(base.forward()).copy()
    empty_wl = W.Workload(**{**wl.__dict__, "a_expert": np.zeros(0, np.int32),
                             "a_src": np.zeros(0, np.int32), "a_dst": np.zeros(0, np.int32),
                             "a_w": np.zeros(0, np.float32)})
    d0 = L.DeviceLayer(empty_wl, weights=(base.w13, base.w2), arithmetic=arithmetic)
    got0 = host(d0.forward())
    assert d0.device_error() == 0
    assert not got0.any()
    wide = W.Workload(**{**wl.__dict__, "T": wl.T + 3})       # three tokens with no rows
    d1 = L.DeviceLayer(wide, weights=(base.w13, base.w2), arithmetic=arithmetic)
    got1 = host(d1.forward())
    assert d1.device_error() == 0
    assert np.array_equal(got1[:wl.T], want)
    assert not got1[wl.T:].any()


def test_layer_at_the_largest_hidden_size(lib):
    """H = 8192, the largest the row kernels and the layer accept: the w13 GEMM stages
    16 rows of 4.5 KiB (more than 64 KiB of LDS) and w2 has N = 8192."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("layer H=8192")
    wl = W.make_workload("ragged570", E=6, H=8192, I=256)
    dl = L.DeviceLayer(wl)
    got = host(dl.forward()).view(np.uint16).copy()
    assert dl.device_error() == 0
    want = omoe.layer_forward(wl.x, wl.a_expert, wl.a_src, wl.a_dst, wl.a_w, wl.T, wl.w13, wl.w2,
                              wl.g_gate, wl.g_up, wl.g_down, wl.E, wl.H, wl.I)
    frac, worst = _e2e_ok(got, want)
    say("H=8192: fraction within tolerance %.5f, worst %.4f x RMS" % (frac, worst))
    assert frac >= E2E_FRAC


# ------------------------------------------------------------------------------ full size
def _pick_tokens(wl, name):
    counts = np.bincount(wl.a_dst, minlength=wl.T)
    if name == "decode1":
        return [0]
    if name.startswith("decode"):
        return [0, wl.T - 1]
    if name == "ragged570":
        return [int(np.argmin(counts))]
    if name == "ragged2303":
        return [0, wl.T - 1]
    hot = int(np.argmax(np.bincount(wl.a_expert, minlength=wl.E)))
    t_hot = int(wl.a_dst[np.where(wl.a_expert == hot)[0][0]])
    return sorted({t_hot, 5})


@pytest.mark.parametrize("name", ["decode1", "ragged570", "ragged2303", "zipf512", "decode4",
                                  "decode32"])
def test_full_size_layer_sampled_tokens(lib, full_weights, name):
    """The full-size workloads in the launch configuration the benchmark times; the
    oracle recomputes a few whole output rows (every row of those tokens)."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload(name)
    say("full-size layer", name, "R=%d" % wl.R)
    dl = L.DeviceLayer(wl, weights=full_weights)
    got = host(dl.forward()).view(np.uint16).copy()
    assert dl.device_error() == 0
    again = host(dl.forward()).view(np.uint16)
    assert np.array_equal(again, got)                       # deterministic
    tokens = _pick_tokens(wl, name)
    say("oracle for tokens", tokens)
    want = _oracle_tokens(wl, tokens)
    frac, worst = _e2e_ok(got[tokens], want)
    say("%s: fraction within tolerance %.5f, worst %.4f x RMS" % (name, frac, worst))
    assert frac >= E2E_FRAC


# ------------------------------------------------------------------------------ HIP graph
@pytest.mark.parametrize("name", ["decode1", "decode8", "ragged570", "ragged2303", "zipf512"])
def test_full_size_w4a16_sampled_tokens(lib, full_weights, name):
    """moe_layer_forward_w4a16 at full size on the resident expert set; the W4A16 oracle
    recomputes every row of a few tokens."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload(name)
    say("full-size W4A16 layer", name, "R=%d" % wl.R)
    dl = L.DeviceLayer(wl, weights=full_weights, arithmetic="w4a16")
    got = host(dl.forward()).view(np.uint16).copy()
    assert dl.device_error() == 0
    tokens = _pick_tokens(wl, name)
    sel = np.where(np.isin(wl.a_dst, tokens))[0]
    want = omoe.layer_forward_w4a16(wl.x, wl.a_expert[sel], wl.a_src[sel], wl.a_dst[sel],
                                    wl.a_w[sel], wl.T, wl.w13, wl.w2, wl.g_gate, wl.g_up,
                                    wl.g_down, wl.E, wl.H, wl.I)[tokens]
    frac, worst = _e2e_ok(got[tokens], want)
    say("%s W4A16: fraction within tolerance %.5f, worst %.4f x RMS" % (name, frac, worst))
    assert frac >= E2E_FRAC


def test_graph_replay_matches_eager(lib):
    """A captured layer replays to the eager output bit for bit, replay after replay, with
    eager work between replays (no memset nodes are recorded: the flags of the one-launch
    GEMM pair, in the last two cases on its large and its small grid, are cleared by the
    grouping kernel)."""
    import torch
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    for name, dims in (("tiny", {}), ("ragged570", dict(E=32, H=512, I=256)),
                       ("zipf512", dict(E=48, H=256, I=256)),
                       ("decode2", dict(E=32, H=512, I=1024)),
                       ("ragged570", dict(E=160, H=4096, I=1024)), ("decode8", {})):
        say("graph", name, dims)
        wl = W.make_workload(name, **dims)
        dl = L.DeviceLayer(wl, experts=wl.active_experts())
        want = dl.forward().clone()
        sync()
        graph = dl.capture_graph()
        for rep in range(4):
            dl.out.zero_()
            graph.replay()
            sync()
            assert torch.equal(dl.out, want), (name, rep)
            dl.forward()  # eager launches between replays
            sync()
            assert torch.equal(dl.out, want), (name, rep)
        assert dl.device_error() == 0
