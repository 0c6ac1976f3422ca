"""GPU parity at the full layer size (288 experts, H=4096, I=2048), in the launch
configurations the benchmark times.

* The grouped GEMM's large-grid instances (one workgroup per (expert, 8 tiles), two tiles
  per wave, 4-chunk weight ring, 8-chunk scale groups) against the oracle at the GEMM
  tolerance, on the real resident weights: w13 (N = 4096, K = 4096) over the 570- and
  2303-row batches' groups and w2 (N = 4096, K = 2048) over the 2303-row groups (a group
  of 18 rows takes two passes).  Every row is compared on 256 columns spread over every
  tile position of a work item (the oracle computes only those weight rows).
* The small-grid instance (8-chunk ring, one tile per wave) against the large-grid one,
  bit for bit, at K = 4096, where the two rings really differ.
* The fused layer against the seven entry points called one by one, bit for bit, on the
  full-size workloads (the large-grid SwiGLU epilogue and scatter-ready epilogue, the
  decode-sized launches that group and quantize inside the GEMMs), and at H = I = 8192 on
  a decode-sized batch (the in-GEMM quantizer's second block per thread).

[GG] is the page "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1
included, so the crossover is 1" (gabewillen.github.io/rocket); section "Proof" runs the
kernel checks against CPU references, fused against separate, and determinism.
"""
import numpy as np
import pytest

from oracle import moe as omoe
from oracle import nvfp4 as onv

from gpu_helpers import composed_layer, dev, empty, host, offsets_from_sizes, say, sync

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3
N_FULL = 4096
# 16 of the 256 tiles: every 16th, shifted so that each of the 8 tile positions of a
# large-grid work item (4 waves x 2 tiles) is covered twice
SAMPLE_TILES = [16 * i + (i % 8) for i in range(16)]
SAMPLE_COLS = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in SAMPLE_TILES])


def _grouped(wl):
    """The oracle's grouping of a workload: offsets and the source row of each grouped row."""
    g = omoe.group_rows(wl.a_expert, wl.a_src, wl.a_dst, wl.a_w, wl.E, wl.S, wl.T)
    return g["offsets"], g["row_src"]


def _oracle_cols(aq, as_, offsets, weight_fn, K):
    """The oracle GEMM restricted to the sampled output columns (their weight rows)."""
    sub = lambda e: tuple(a[SAMPLE_COLS] for a in weight_fn(e))
    return omoe.grouped_gemm(aq, as_, offsets, sub, len(SAMPLE_COLS), K)


def _gemm(B, aq, as_, offsets, w, N, K):
    import torch
    R = aq.shape[0]
    out = torch.full((R, N), float("nan"), dtype=torch.float32, device="cuda")
    B.grouped_gemm_nvfp4(dev(aq), dev(as_), dev(offsets), len(offsets) - 1, R, w, N, K, out,
                         B.MOE_PATH_AUTO, 0)
    sync()
    return host(out)


def _check_tol(got_cols, want):
    rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
    err = np.abs(got_cols - want)
    assert np.all(np.isfinite(got_cols))
    worst = float((err / rms).max())
    say("worst |gpu - oracle| / row RMS = %.3g" % worst)
    assert np.all(err <= GEMM_TOL * rms), worst


@pytest.fixture(scope="module")
def w13_ragged570(lib, full_weights):
    """The w13 GEMM over ragged570's groups (oracle-quantized rows), large-grid instance."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload("ragged570")
    offsets, row_src = _grouped(wl)
    xq, xs, _ = onv.quantize_rows(onv.bf16_bits_to_f32(wl.x[row_src]))
    got = _gemm(B, xq, xs, offsets, full_weights[0], N_FULL, wl.H)
    return wl, offsets, xq, xs, got


@pytest.mark.parametrize("name", ["ragged570", "ragged2303"])
def test_w13_large_grid_against_oracle(lib, full_weights, w13_ragged570, name):
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("full-size w13 GEMM vs oracle", name)
    if name == "ragged570":
        wl, offsets, xq, xs, got = w13_ragged570
    else:
        wl = W.make_workload(name)
        offsets, row_src = _grouped(wl)
        xq, xs, _ = onv.quantize_rows(onv.bf16_bits_to_f32(wl.x[row_src]))
        got = _gemm(B, xq, xs, offsets, full_weights[0], N_FULL, wl.H)
    assert int(offsets[-1]) == wl.R and (np.diff(offsets) > 0).all()   # 288 groups
    want = _oracle_cols(xq, xs, offsets, wl.w13, wl.H)
    _check_tol(got[:, SAMPLE_COLS], want)


def test_w2_large_grid_against_oracle(lib, full_weights):
    """K = I = 2048 over ragged2303's groups (sizes 1..18: one group takes two passes, its
    weights loaded through the caches); activations are random rows quantized by the
    oracle."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("full-size w2 GEMM vs oracle")
    wl = W.make_workload("ragged2303")
    offsets, _ = _grouped(wl)
    assert np.diff(offsets).max() > 16
    rows = W.bf16_normal(77, (wl.R, wl.I), 5)
    hq, hs, _ = onv.quantize_rows(onv.bf16_bits_to_f32(rows))
    got = _gemm(B, hq, hs, offsets, full_weights[1], N_FULL, wl.I)
    want = _oracle_cols(hq, hs, offsets, wl.w2, wl.I)
    _check_tol(got[:, SAMPLE_COLS], want)


def test_grid_instances_agree_bitwise_at_k4096(lib, full_weights, w13_ragged570):
    """Three experts' rows alone (the small-grid instance: 8-chunk ring, one tile per wave)
    give the bits of the same rows in the 288-group launch (the large-grid instance: 4-chunk
    ring, two tiles per wave), at K = 4096 where the scale group is 8 chunks."""
    from nvfp4_block_scaled_gather_amd import binding as B
    say("grid instances bitwise at K=4096")
    wl, offsets, xq, xs, big = w13_ragged570
    pick = [0, 143, 287]
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in pick])
    sizes = np.zeros(wl.E, np.int64)
    sizes[pick] = np.diff(offsets)[pick]
    small = _gemm(B, xq[rows], xs[rows], offsets_from_sizes(sizes), full_weights[0], N_FULL, wl.H)
    assert np.array_equal(small.view(np.uint32), big[rows].view(np.uint32))


@pytest.mark.parametrize("name", ["decode1", "decode2", "decode4", "decode8", "ragged570",
                                  "ragged2303", "zipf512"])
def test_full_size_layer_equals_separate_calls(lib, full_weights, name):
    """moe_layer_forward at full size equals the separate entry points bit for bit: the
    decode-sized launches (8 and 16 assignments: two launches, the w2 launch summing the
    tokens; 32: grouping and quantization inside the GEMMs, then the per-token sum),
    the five-launch path with small-grid (64 rows) and large-grid GEMMs, and the Zipf batch's
    multi-pass groups."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload(name)
    say("full-size layer vs separate calls", name, "R=%d" % wl.R)
    dl = L.DeviceLayer(wl, weights=full_weights)
    got = host(dl.forward()).copy()
    assert dl.device_error() == 0
    assert np.array_equal(got, composed_layer(B, dl, B.MOE_PATH_AUTO, 0))


# group sizes of the one-launch GEMM pair's test batch: multi-pass groups (double passes,
# a single pass after them, four quantization parts), one exactly 16 rows, small groups
ONE_LAUNCH_SIZES = [61, 41, 33, 17, 16, 12, 9, 5, 3, 2, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1]
ONE_LAUNCH_EXPERTS = [3, 150, 77, 11, 42, 99, 5, 120, 60, 159, 0, 1, 2, 40, 41, 100, 101, 130,
                      131, 149]


def _one_launch_batch(base, case):
    """Assignments of `base` (its first R) moved onto chosen experts, in a shuffled order:
    "groups": ONE_LAUNCH_SIZES rows on ONE_LAUNCH_EXPERTS; "edge": 65 groups of one row
    (the smallest batch whose grid is large at these sizes); "small": 40 rows in 9 groups
    (a small grid: the decode instances); "invalid": "groups" with two
    expert ids and one output row out of range (dropped, error bits set)."""
    from nvfp4_block_scaled_gather_amd import workloads as W
    if case == "edge":
        a_expert = np.arange(0, 2 * 65, 2, dtype=np.int32)
    elif case == "small":
        a_expert = np.repeat(np.asarray(ONE_LAUNCH_EXPERTS[:9], np.int32),
                             [17, 9, 5, 3, 2, 1, 1, 1, 1])
    else:
        a_expert = np.repeat(np.asarray(ONE_LAUNCH_EXPERTS, np.int32), ONE_LAUNCH_SIZES)
    R = len(a_expert)
    np.random.default_rng(7).shuffle(a_expert)
    a_dst = base.a_dst[:R].copy()
    if case == "invalid":
        a_expert[[4, 90]] = [base.E, -1]
        a_dst[17] = base.T
    return W.Workload(**{**base.__dict__, "a_expert": a_expert, "a_src": base.a_src[:R],
                         "a_dst": a_dst, "a_w": base.a_w[:R]})


@pytest.mark.parametrize("I,case", [(1024, "groups"), (2048, "groups"), (2048, "edge"),
                                    (2048, "small"), (2048, "invalid")])
def test_one_launch_gemm_pair_equals_separate_calls(lib, full_weights, I, case):
    """A batch of more than 32 assignments (H and I multiples of 1024, I <= 2048) runs the
    w13 GEMM, the quantization of h and the w2 GEMM in one launch: the
    w13 items flag their parts of h, four quantization workgroups per group wait for the
    group's flags, and the w2 items wait for their group's quantization ([MF], the fusion of
    the two grouped GEMMs).  Bit-identical to the separate entry points, twice in a row (the
    flags are cleared for each call): groups of 1 to 61 rows on 20 of E experts, with one
    (I = 1024) and two (I = 2048) scale blocks per lane in the quantization of h; 65 groups
    of one row (the smallest batch on the large grid); 40 rows (a small grid); dropped
    assignments (their error bits, and never MOE_ERR_SYNC, which a wait that gave up would
    set)."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    E = 288 if I == 2048 else 160
    base = W.make_workload("ragged570", E=E, H=4096, I=I)
    wl = _one_launch_batch(base, case)
    say("one-launch GEMM pair vs separate calls", case, "E=%d I=%d R=%d" % (E, I, wl.R))
    assert wl.R > 32
    weights = full_weights if I == 2048 else None
    dl = L.DeviceLayer(wl, flags=0, gemv_max_rows=0, weights=weights,
                       experts=None if weights else wl.active_experts())
    want = composed_layer(B, dl, 0, 0)
    err_want = B.MOE_ERR_EXPERT | B.MOE_ERR_DST if case == "invalid" else 0
    for rep in range(2):
        got = host(dl.forward()).copy()
        assert dl.device_error() == err_want
        assert np.array_equal(got, want), rep


@pytest.mark.parametrize("name", ["decode1", "decode4"])
def test_widest_decode_layer_equals_separate_calls(lib, name):
    """H = I = 8192 on a decode-sized batch: the quantizer inside each GEMM launch gives
    each thread two 16-element blocks of a row (512 blocks on 256 threads), for x in the w13
    launch and for h in the w2 launch; bit-identical to the separate entry points."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    wl = W.make_workload(name, E=8, H=8192, I=8192)
    say("H=I=8192 decode-sized layer vs separate calls", name, "R=%d" % wl.R)
    assert wl.R <= 32
    dl = L.DeviceLayer(wl)
    got = host(dl.forward()).copy()
    assert dl.device_error() == 0
    assert np.array_equal(got, composed_layer(B, dl, B.MOE_PATH_AUTO, 0))
    assert np.count_nonzero(got) > 0.9 * got.size
