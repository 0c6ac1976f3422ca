"""ctypes binding of libmoe_nvfp4.so (the C ABI in include/moe_nvfp4.h).

Argument marshalling only: each function has the C entry point's name, takes torch
tensors (device memory) in place of pointers, passes the current HIP stream, and raises
``MoeError`` on a non-zero status.  Every step of the layer runs in the HIP library;
there is no fallback path — a missing or stale library is an error.
"""
import ctypes
import os

from . import build as _build

LIB_PATH = _build.LIB_PATH

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EHIP = -3
MOE_EWORKSPACE = -4
MOE_PATH_AUTO = 0
MOE_PATH_FORCE_GEMV = 1
MOE_PATH_FORCE_MFMA = 2
MOE_ERR_EXPERT = 1
MOE_ERR_SRC = 2
MOE_ERR_DST = 4
MOE_ERR_SYNC = 8

# Default largest group on the GEMV path under MOE_PATH_AUTO.  Measured on MI355X, the MFMA
# path streams the weights faster than the GEMV path for every group size, one row included,
# so by default every group takes the MFMA path; the GEMV path stays selectable.
DEFAULT_GEMV_MAX_ROWS = 0


class MoeError(RuntimeError):
    def __init__(self, name, code, text):
        super().__init__("%s failed with status %d: %s" % (name, code, text))
        self.code = code


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("w13_packed", ctypes.c_void_p), ("w2_packed", ctypes.c_void_p),
                ("g_gate", ctypes.c_void_p), ("g_up", ctypes.c_void_p),
                ("g_down", ctypes.c_void_p), ("flags", ctypes.c_int),
                ("gemv_max_rows", ctypes.c_int)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = {
    "nvfp4_packed_weight_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "nvfp4_pack_weights": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "nvfp4_unpack_weights": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_gather_rows": (_I, [_P, _I, _I, _P, _P, _P, _P, _I, _I, _I,
                             _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_rows": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "grouped_gemm_nvfp4": (_I, [_P, _P, _P, _I, _I, _P, _I, _I, _P, _I, _I, _P]),
    "grouped_gemm_w4a16": (_I, [_P, _P, _I, _I, _P, _I, _I, _P, _P]),
    "swiglu_grouped": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "moe_scatter_add": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P, _P, _I, _P, _P]),
    "moe_layer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MoeLayerDesc), _I, _I, _I]),
    "moe_layer_forward": (_I, [ctypes.POINTER(MoeLayerDesc), _P, _I, _P, _P, _P, _P, _I, _I,
                               _P, _P, ctypes.c_size_t, _P]),
    "moe_layer_forward_w4a16": (_I, [ctypes.POINTER(MoeLayerDesc), _P, _I, _P, _P, _P, _P, _I,
                                     _I, _P, _P, ctypes.c_size_t, _P]),
    "moe_layer_forward_noalloc": (_I, [ctypes.POINTER(MoeLayerDesc), _P, _I, _P, _P, _P, _P, _I,
                                       _I, _P, _P, _P]),
    "moe_hbm_read_probe": (_I, [_P, ctypes.c_size_t, _I, ctypes.c_uint32, _P, _P]),
    "moe_hbm_read_probe_variants": (_I, []),
    "moe_get_device_error": (_I, [_P, _P]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_source_hash": (ctypes.c_char_p, []),
}

_lib = None


def load(check_fresh=True):
    """Load the library (once).  Refuses a build whose source hash differs from the
    sources on disk: a stale binary would silently test something else."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("HIP library %s is not built: run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if check_fresh:
        built = lib.moe_source_hash().decode()
        now = _build.source_hash()
        if built != now:
            raise RuntimeError("HIP library %s is stale (built from %s, sources are %s): rebuild it"
                               % (LIB_PATH, built, now))
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(name, rc):
    if rc != MOE_OK:
        raise MoeError(name, rc, load().moe_last_error().decode())


# ----------------------------------------------------------------------------- entry points
def nvfp4_packed_weight_bytes(E, N, K):
    return int(load().nvfp4_packed_weight_bytes(E, N, K))


def nvfp4_pack_weights(nib, scl, E, N, K, packed, stream=None):
    _check("nvfp4_pack_weights",
           load().nvfp4_pack_weights(_ptr(nib), _ptr(scl), E, N, K, _ptr(packed), _stream(stream)))


def nvfp4_unpack_weights(packed, E, N, K, nib, scl, stream=None):
    _check("nvfp4_unpack_weights",
           load().nvfp4_unpack_weights(_ptr(packed), E, N, K, _ptr(nib), _ptr(scl), _stream(stream)))


def moe_gather_rows(x, S, H, a_expert, a_src, a_dst, a_w, R, E, T, xg, expert_offsets,
                    row_src, row_dst, row_w, tok_off, tok_rows, err_word, stream=None):
    _check("moe_gather_rows", load().moe_gather_rows(
        _ptr(x), S, H, _ptr(a_expert), _ptr(a_src), _ptr(a_dst), _ptr(a_w), R, E, T, _ptr(xg),
        _ptr(expert_offsets), _ptr(row_src), _ptr(row_dst), _ptr(row_w), _ptr(tok_off),
        _ptr(tok_rows), _ptr(err_word), _stream(stream)))


def nvfp4_quantize_rows(inp, R, K, q, sc, row_gs, stream=None):
    _check("nvfp4_quantize_rows", load().nvfp4_quantize_rows(
        _ptr(inp), R, K, _ptr(q), _ptr(sc), _ptr(row_gs), _stream(stream)))


def grouped_gemm_nvfp4(aq, as_, expert_offsets, E, R, w_packed, N, K, out,
                       flags=MOE_PATH_AUTO, gemv_max_rows=DEFAULT_GEMV_MAX_ROWS, stream=None):
    _check("grouped_gemm_nvfp4", load().grouped_gemm_nvfp4(
        _ptr(aq), _ptr(as_), _ptr(expert_offsets), E, R, _ptr(w_packed), N, K, _ptr(out),
        flags, gemv_max_rows, _stream(stream)))


def grouped_gemm_w4a16(a, expert_offsets, E, R, w_packed, N, K, out, stream=None):
    _check("grouped_gemm_w4a16", load().grouped_gemm_w4a16(
        _ptr(a), _ptr(expert_offsets), E, R, _ptr(w_packed), N, K, _ptr(out), _stream(stream)))


def swiglu_grouped(acc13, R, I, expert_offsets, E, g_gate, g_up, row_gs, h, stream=None):
    _check("swiglu_grouped", load().swiglu_grouped(
        _ptr(acc13), R, I, _ptr(expert_offsets), E, _ptr(g_gate), _ptr(g_up), _ptr(row_gs),
        _ptr(h), _stream(stream)))


def moe_scatter_add(y, R, H, expert_offsets, E, row_w, g_down, row_gs, tok_off, tok_rows, T,
                    out, stream=None):
    _check("moe_scatter_add", load().moe_scatter_add(
        _ptr(y), R, H, _ptr(expert_offsets), E, _ptr(row_w), _ptr(g_down), _ptr(row_gs),
        _ptr(tok_off), _ptr(tok_rows), T, _ptr(out), _stream(stream)))


def make_layer_desc(E, H, I, w13_packed, w2_packed, g_gate, g_up, g_down,
                    flags=MOE_PATH_AUTO, gemv_max_rows=DEFAULT_GEMV_MAX_ROWS):
    return MoeLayerDesc(E, H, I, w13_packed.data_ptr(), w2_packed.data_ptr(), g_gate.data_ptr(),
                        g_up.data_ptr(), g_down.data_ptr(), flags, gemv_max_rows)


def moe_layer_workspace_bytes(desc, S, R, T):
    return int(load().moe_layer_workspace_bytes(ctypes.byref(desc), S, R, T))


def moe_layer_forward(desc, x, S, a_expert, a_src, a_dst, a_w, R, T, out, workspace,
                      workspace_bytes, stream=None):
    _check("moe_layer_forward", load().moe_layer_forward(
        ctypes.byref(desc), _ptr(x), S, _ptr(a_expert), _ptr(a_src), _ptr(a_dst), _ptr(a_w), R, T,
        _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def moe_layer_forward_w4a16(desc, x, S, a_expert, a_src, a_dst, a_w, R, T, out, workspace,
                            workspace_bytes, stream=None):
    _check("moe_layer_forward_w4a16", load().moe_layer_forward_w4a16(
        ctypes.byref(desc), _ptr(x), S, _ptr(a_expert), _ptr(a_src), _ptr(a_dst), _ptr(a_w), R, T,
        _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def moe_hbm_read_probe(src, nbytes, variant, key, sink, stream=None):
    _check("moe_hbm_read_probe", load().moe_hbm_read_probe(
        _ptr(src), nbytes, variant, key, _ptr(sink), _stream(stream)))


def moe_hbm_read_probe_variants():
    return int(load().moe_hbm_read_probe_variants())


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_layer_forward_noalloc(desc, x, S, a_expert, a_src, a_dst, a_w, R, T, out, err_word=None,
                              stream=None):
    _check("moe_layer_forward_noalloc", load().moe_layer_forward_noalloc(
        ctypes.byref(desc), _ptr(x), S, _ptr(a_expert), _ptr(a_src), _ptr(a_dst), _ptr(a_w), R, T,
        _ptr(out), _ptr(err_word), _stream(stream)))


def moe_get_device_error(err_word, stream=None):
    rc = load().moe_get_device_error(_ptr(err_word), _stream(stream))
    if rc < 0:
        _check("moe_get_device_error", rc)
    return rc
