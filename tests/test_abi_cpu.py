"""Host-side checks of the C ABI that need no GPU: the built library loads, exports every
function the public header declares, and rejects bad arguments before launching.

[GG] is the page "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1
included, so the crossover is 1"; [MF] the page "Fusing the MoE layer's two grouped GEMMs is
worth 4%, and a CUDA graph already collects it" (gabewillen.github.io/rocket).
"""
import ctypes
import os
import re

import pytest

from nvfp4_block_scaled_gather_amd import binding as B
from nvfp4_block_scaled_gather_amd import build as build_mod
from nvfp4_block_scaled_gather_amd import layer as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_header_declares_the_layer_entry_points():
    names = _declared_functions()
    for n in ("moe_gather_rows", "nvfp4_quantize_rows", "grouped_gemm_nvfp4", "swiglu_grouped",
              "moe_scatter_add", "moe_layer_forward", "nvfp4_pack_weights"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(B._SIGNATURES), "binding and header disagree"


def test_library_is_fresh(lib):
    assert lib.moe_source_hash().decode() == build_mod.source_hash()


def test_packed_bytes_follow_the_page_byte_model(lib):
    """Table "Bytes decide it before the kernel runs" ([MF]): 288 experts,
    w13 = 288*4096*4096*(0.5+1/16) = 2.718 GB, w2 = 1.359 GB, 4.077 GB total, a 13.5 MiB
    expert, 17.13 ms at 238 GB/s."""
    g = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "byte_model.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            g[k] = float(v)
    E, H, I = int(g["experts"]), int(g["hidden"]), int(g["intermediate"])
    w13 = B.nvfp4_packed_weight_bytes(E, 2 * I, H)
    w2 = B.nvfp4_packed_weight_bytes(E, H, I)
    assert round(w13 / 1e9, 3) == g["w13_GB"]
    assert round(w2 / 1e9, 3) == g["w2_GB"]
    assert round((w13 + w2) / 1e9, 3) == g["total_GB"]
    assert (w13 + w2) / E / 2 ** 20 == g["slot_MiB"]
    assert round((w13 + w2) / (g["roofline_GBps"] * 1e9) * 1e3, 2) == g["roofline_ms"]
    assert L.weight_stream_bytes(E, H, I) == w13 + w2


def _status(rc):
    return rc


def test_argument_errors_are_reported_before_launch(lib):
    null = None
    # unsupported shapes
    assert lib.nvfp4_packed_weight_bytes(1, 17, 128) == 0
    assert lib.nvfp4_packed_weight_bytes(1, 16, 100) == 0
    assert lib.nvfp4_pack_weights(null, null, 1, 16, 100, null, null) == B.MOE_EUNSUPPORTED
    assert lib.nvfp4_pack_weights(null, null, 1, 16, 128, null, null) == B.MOE_EINVAL
    assert b"null" in lib.moe_last_error()
    # GEMM: bad K, bad N, bad flags, misaligned pointers
    p16 = ctypes.c_void_p(4096)
    assert lib.grouped_gemm_nvfp4(p16, p16, p16, 8, 4, p16, 64, 100, p16, 0, 4, null) == B.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_nvfp4(p16, p16, p16, 8, 4, p16, 60, 128, p16, 0, 4, null) == B.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_nvfp4(p16, p16, p16, 8, 4, p16, 64, 128, p16, 7, 4, null) == B.MOE_EINVAL
    assert lib.grouped_gemm_nvfp4(p16, p16, p16, 8, 4, p16, 64, 128, p16, 0, -1, null) == B.MOE_EINVAL
    p8 = ctypes.c_void_p(4096 + 8)
    assert lib.grouped_gemm_nvfp4(p8, p16, p16, 8, 4, p16, 64, 128, p16, 0, 4, null) == B.MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()
    assert lib.grouped_gemm_nvfp4(p16, p16, p16, 0, 4, p16, 64, 128, p16, 0, 4, null) == B.MOE_EUNSUPPORTED
    # quantize: K not a multiple of 16 / too large; nulls
    assert lib.nvfp4_quantize_rows(p16, 4, 24, p16, p16, p16, null) == B.MOE_EUNSUPPORTED
    assert lib.nvfp4_quantize_rows(p16, 4, 16384, p16, p16, p16, null) == B.MOE_EUNSUPPORTED
    assert lib.nvfp4_quantize_rows(null, 4, 64, p16, p16, p16, null) == B.MOE_EINVAL
    assert lib.nvfp4_quantize_rows(p16, -1, 64, p16, p16, p16, null) == B.MOE_EINVAL
    # gather / group
    assert lib.moe_gather_rows(p16, 4, 64, p16, p16, p16, p16, 4, 8, 20000, p16, p16, p16, p16, p16,
                               p16, p16, p16, null) == B.MOE_EUNSUPPORTED
    assert lib.moe_gather_rows(p16, 4, 64, null, p16, p16, p16, 4, 8, 4, p16, p16, p16, p16, p16,
                               p16, p16, p16, null) == B.MOE_EINVAL
    assert lib.moe_gather_rows(p16, 4, 60, p16, p16, p16, p16, 4, 8, 4, p16, p16, p16, p16, p16,
                               p16, p16, p16, null) == B.MOE_EUNSUPPORTED
    # swiglu / scatter
    assert lib.swiglu_grouped(p16, 4, 24, p16, 8, p16, p16, p16, p16, null) == B.MOE_EUNSUPPORTED
    assert lib.moe_scatter_add(p16, 4, 6, p16, 8, p16, p16, p16, p16, p16, 2, p16, null) == B.MOE_EUNSUPPORTED
    # layer: bad H, small workspace, null descriptor
    d = B.MoeLayerDesc(8, 256, 128, 4096, 4096, 4096, 4096, 4096, 0, 4)
    need = lib.moe_layer_workspace_bytes(ctypes.byref(d), 4, 8, 4)
    assert need > 0
    ws = ctypes.c_void_p(1 << 20)
    assert lib.moe_layer_forward(ctypes.byref(d), p16, 4, p16, p16, p16, p16, 8, 4, p16, ws,
                                 need - 1, null) == B.MOE_EWORKSPACE
    bad = B.MoeLayerDesc(8, 200, 128, 4096, 4096, 4096, 4096, 4096, 0, 4)
    assert lib.moe_layer_workspace_bytes(ctypes.byref(bad), 4, 8, 4) == 0
    assert lib.moe_layer_forward(ctypes.byref(bad), p16, 4, p16, p16, p16, p16, 8, 4, p16, ws,
                                 need, null) == B.MOE_EUNSUPPORTED
    assert lib.moe_layer_forward(None, p16, 4, p16, p16, p16, p16, 8, 4, p16, ws, need, null) == B.MOE_EINVAL
    assert lib.moe_get_device_error(null, null) == B.MOE_EINVAL
    # h's NVFP4 rows (R x I/2 bytes) beyond the GEMM's 32-bit staging range, while x's rows
    # (R x H/2) are not: refused before any launch instead of wrapping the offsets
    narrow = B.MoeLayerDesc(8, 128, 8192, 4096, 4096, 4096, 4096, 4096, 0, 0)
    R_big = 600000
    assert R_big * 128 < (1 << 31) <= R_big * 8192
    assert lib.moe_layer_workspace_bytes(ctypes.byref(narrow), 4, R_big, 4) == 0
    assert lib.moe_layer_forward(ctypes.byref(narrow), p16, 4, p16, p16, p16, p16, R_big, 4, p16,
                                 ws, 1 << 40, null) == B.MOE_EUNSUPPORTED
    assert b"rows of h" in lib.moe_last_error()
    # W4A16: K beyond what the staged bf16 rows fit in LDS, misalignment, H above 4096
    assert lib.grouped_gemm_w4a16(p16, p16, 8, 4, p16, 64, 8192, p16, null) == B.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_w4a16(p16, p16, 8, 4, p16, 64, 100, p16, null) == B.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_w4a16(p8, p16, 8, 4, p16, 64, 128, p16, null) == B.MOE_EINVAL
    wide = B.MoeLayerDesc(8, 8192, 128, 4096, 4096, 4096, 4096, 4096, 0, 0)
    wneed = lib.moe_layer_workspace_bytes(ctypes.byref(wide), 4, 8, 4)
    assert wneed > 0
    assert lib.moe_layer_forward_w4a16(ctypes.byref(wide), p16, 4, p16, p16, p16, p16, 8, 4, p16,
                                       ws, wneed, null) == B.MOE_EUNSUPPORTED
    assert lib.moe_layer_forward_w4a16(ctypes.byref(d), p16, 4, p16, p16, p16, p16, 8, 4, p16, ws,
                                       need - 1, null) == B.MOE_EWORKSPACE


def test_read_probe_rejects_bad_arguments_before_launch(lib):
    p16 = ctypes.c_void_p(4096)
    n = lib.moe_hbm_read_probe_variants()
    assert n == 5
    unit = 294912
    assert lib.moe_hbm_read_probe(p16, unit + 16, 0, 0, p16, None) == B.MOE_EUNSUPPORTED
    assert lib.moe_hbm_read_probe(p16, 0, 0, 0, p16, None) == B.MOE_EUNSUPPORTED
    assert lib.moe_hbm_read_probe(p16, unit, n, 0, p16, None) == B.MOE_EINVAL
    assert lib.moe_hbm_read_probe(p16, unit, -1, 0, p16, None) == B.MOE_EINVAL
    assert lib.moe_hbm_read_probe(None, unit, 0, 0, p16, None) == B.MOE_EINVAL
    assert lib.moe_hbm_read_probe(ctypes.c_void_p(4104), unit, 0, 0, p16, None) == B.MOE_EINVAL


def test_noalloc_layer_rejects_oversized_calls_before_any_device_call(lib):
    """moe_layer_forward_noalloc refuses a call whose workspace exceeds its fixed scratch
    array (and bad arguments) on the host, before it looks up the array on a device."""
    p16 = ctypes.c_void_p(4096)
    d = B.MoeLayerDesc(288, 4096, 2048, 4096, 4096, 4096, 4096, 4096, 0, 0)
    big = 2900
    assert lib.moe_layer_workspace_bytes(ctypes.byref(d), big, big, 288) > B.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_layer_forward_noalloc(ctypes.byref(d), p16, big, p16, p16, p16, p16, big, 288,
                                         p16, None, None) == B.MOE_EUNSUPPORTED
    assert b"scratch" in lib.moe_last_error()
    assert lib.moe_layer_forward_noalloc(None, p16, 4, p16, p16, p16, p16, 8, 4, p16, None,
                                         None) == B.MOE_EINVAL
    assert lib.moe_layer_forward_noalloc(ctypes.byref(d), p16, 4, p16, p16, p16, p16, 8, 4, p16,
                                         ctypes.c_void_p(4098), None) == B.MOE_EINVAL
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == B.MOE_NOALLOC_SCRATCH_BYTES


def test_workspace_grows_with_rows(lib):
    d = B.MoeLayerDesc(288, 4096, 2048, 4096, 4096, 4096, 4096, 4096, 0, 4)
    a = lib.moe_layer_workspace_bytes(ctypes.byref(d), 570, 570, 8)
    b = lib.moe_layer_workspace_bytes(ctypes.byref(d), 2303, 2303, 288)
    assert 0 < a < b
    # dominated by the fp32 GEMM outputs: R * 2I * 4 bytes
    assert b >= 2303 * 2 * 2048 * 4
