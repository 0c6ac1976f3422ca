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


def composed_layer(B, dl, flags, gemv_max):
    """The layer's steps as separate ABI calls (gather, quantize, w13 GEMM, SwiGLU,
    quantize, w2 GEMM, scatter-add), on the layer's resident inputs; returns out [T, H]."""
    import torch
    wl = dl.wl
    R, E, H, I, T, S = wl.R, wl.E, wl.H, wl.I, wl.T, wl.S
    i32, f32, u8, i16 = torch.int32, torch.float32, torch.uint8, torch.int16
    xg = empty((R, H), i16)
    off = empty((E + 1,), i32)
    rs, rd, rw = empty((R,), i32), empty((R,), i32), empty((R,), f32)
    to, tr, err = empty((T + 1,), i32), empty((R,), i32), empty((1,), i32)
    B.moe_gather_rows(dl.x, S, H, dl.a_expert, dl.a_src, dl.a_dst, dl.a_w, R, E, T, xg, off, rs,
                      rd, rw, to, tr, err)
    xq, xs, xgs = empty((R, H // 2), u8), empty((R, H // 16), u8), empty((R,), f32)
    B.nvfp4_quantize_rows(xg, R, H, xq, xs, xgs)
    acc = empty((R, 2 * I), f32)
    B.grouped_gemm_nvfp4(xq, xs, off, E, R, dl.w13, 2 * I, H, acc, flags, gemv_max)
    h = empty((R, I), i16)
    B.swiglu_grouped(acc, R, I, off, E, dl.g_gate, dl.g_up, xgs, h)
    hq, hs, hgs = empty((R, I // 2), u8), empty((R, I // 16), u8), empty((R,), f32)
    B.nvfp4_quantize_rows(h, R, I, hq, hs, hgs)
    y = empty((R, H), f32)
    B.grouped_gemm_nvfp4(hq, hs, off, E, R, dl.w2, H, I, y, flags, gemv_max)
    out = empty((T, H), i16)
    B.moe_scatter_add(y, R, H, off, E, rw, dl.g_down, hgs, to, tr, T, out)
    sync()
    return host(out)
