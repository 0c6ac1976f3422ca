"""Shared helpers of the GPU parity tests (device marshalling, random NVFP4 data)."""
import sys

import numpy as np


def say(*a):
    """Progress line, flushed, so a GPU run names the case it is in."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def sync():
    import torch
    torch.cuda.synchronize()


def rand_nvfp4(rng, rows, K, scale_lo=0x00, scale_hi=0x7E):
    """Random canonical NVFP4 rows: uniform nibbles, uniform scale codes in a range."""
    nib = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    sc = rng.integers(scale_lo, scale_hi + 1, (rows, K // 16)).astype(np.uint8)
    return nib, sc


def pack(binding, nib, scl, E, N, K):
    """Pack canonical [E*N, K/2] / [E*N, K/16] weights on the device."""
    import torch
    nb = binding.nvfp4_packed_weight_bytes(E, N, K)
    out = torch.empty(nb, dtype=torch.uint8, device="cuda")
    binding.nvfp4_pack_weights(dev(nib), dev(scl), E, N, K, out)
    return out


def offsets_from_sizes(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def run_gemm(binding, aq, as_, offsets, wp, N, K, flags, gemv_max=4):
    import torch
    R = aq.shape[0]
    E = len(offsets) - 1
    out = torch.full((max(R, 1), N), float("nan"), dtype=torch.float32, device="cuda")
    binding.grouped_gemm_nvfp4(dev(aq), dev(as_), dev(offsets), E, R, wp, N, K, out, flags, gemv_max)
    sync()
    return host(out)[:R]
