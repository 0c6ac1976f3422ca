"""moe_layer_forward_noalloc (the layer entry point that allocates nothing: its workspace is
a fixed array the library holds on each GPU) against moe_layer_forward, through the C ABI:
the same launches, so the outputs must agree bit for bit.  Each test makes two calls in a
row, the second with a smaller batch, so the second runs on scratch the first left dirty.
"""
import numpy as np
import pytest

from gpu_helpers import empty, host, say, sync

pytestmark = pytest.mark.gpu


def _noalloc(B, dl, err=None):
    import torch
    wl = dl.wl
    out = torch.full((wl.T, wl.H), -1, dtype=torch.int16, device="cuda")
    B.moe_layer_forward_noalloc(dl.desc, dl.x, wl.S, dl.a_expert, dl.a_src, dl.a_dst, dl.a_w,
                                wl.R, wl.T, out, err)
    sync()
    return host(out)


def _with_workspace(dl):
    got = host(dl.forward()).copy()
    sync()
    return got


def _pair(B, dl):
    import torch
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    got = _noalloc(B, dl, err)
    want = _with_workspace(dl)
    assert np.array_equal(got, want)
    assert B.moe_get_device_error(err) == dl.device_error()
    return got


def test_noalloc_equals_workspace_entry_point_small_shapes(lib):
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    big = W.make_workload("ragged570", E=32, H=512, I=256)
    say("noalloc: ragged570-shaped, R=%d" % big.R)
    d1 = L.DeviceLayer(big)
    _pair(B, d1)
    small = W.make_workload("tiny")
    say("noalloc: then tiny, R=%d" % small.R)
    d2 = L.DeviceLayer(small)
    _pair(B, d2)
    # and again the larger one after the smaller (the array keeps the last call's bytes)
    _pair(B, d1)


def test_noalloc_equals_workspace_entry_point_full_size(lib, full_weights):
    """ragged2303 (288 experts, H=4096, I=2048: 55 MB of scratch, the largest headline
    batch) and then single-token decode (the two-launch path) on the resident experts."""
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    for name in ("ragged2303", "decode1"):
        wl = W.make_workload(name)
        say("noalloc: full-size", name, "R=%d" % wl.R)
        dl = L.DeviceLayer(wl, weights=full_weights)
        assert dl.ws_bytes <= B.MOE_NOALLOC_SCRATCH_BYTES
        got = _pair(B, dl)
        assert np.count_nonzero(got) > 0.9 * got.size


def test_noalloc_reports_dropped_assignments_and_accepts_no_error_word(lib):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("noalloc: invalid assignments")
    wl = W.make_workload("tiny")
    bad = W.Workload(**{**wl.__dict__,
                        "a_expert": np.concatenate([wl.a_expert, [wl.E, 1]]).astype(np.int32),
                        "a_src": np.concatenate([wl.a_src, [0, wl.S + 3]]).astype(np.int32),
                        "a_dst": np.concatenate([wl.a_dst, [1, 0]]).astype(np.int32),
                        "a_w": np.concatenate([wl.a_w, [1, 1]]).astype(np.float32)})
    dl = L.DeviceLayer(bad)
    got = _pair(B, dl)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _noalloc(B, dl, err)
    assert B.moe_get_device_error(err) == B.MOE_ERR_EXPERT | B.MOE_ERR_SRC
    assert np.array_equal(_noalloc(B, dl, None), got)


def test_noalloc_rejects_a_batch_beyond_its_scratch(lib):
    import torch
    from nvfp4_block_scaled_gather_amd import binding as B
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    say("noalloc: oversized batch refused")
    wl = W.make_workload("tiny")
    dl = L.DeviceLayer(wl)
    R = 200000   # needs far more than the fixed array at this shape
    big = empty((R,), torch.int32)
    out = empty((wl.T, wl.H), torch.int16)
    with pytest.raises(B.MoeError) as ex:
        B.moe_layer_forward_noalloc(dl.desc, dl.x, wl.S, big, big, big, empty((R,), torch.float32),
                                    R, wl.T, out, None)
    assert ex.value.code == B.MOE_EUNSUPPORTED
