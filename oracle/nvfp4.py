"""NVFP4 codec and row quantizer (CPU oracle; test infrastructure only).

NVFP4, as the pages use it ([MF] table "Bytes decide it before the kernel runs": each
weight costs 0.5 + 1/16 bytes; [MF] "Different globals on the two halves": e4m3 block
scales and an fp32 ``weight_scale_2`` global per projection):

* element: e2m1 nibble — bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
* block scale: one e4m3 byte per 16 consecutive elements along K.  The variant is the
  OCP "e4m3fn" one: [MF] gives the e4m3 grid 126 finite positive codes, which holds for
  e4m3fn (0x7F is NaN, max 448) and not for the FNUZ variant (127 codes, max 240);
* global: one fp32 scale per row (activations) or per projection (weights).

Every value here is built from the bit definitions, and encoders are nearest-value
searches over the decoded grid — no bit tricks — so that a reader can check them by eye.
"""
import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0
# Per-row activation global: gs = amax / (6 * 448), so that the block holding amax gets
# the largest e4m3 scale.  6 is the largest e2m1 magnitude, 448 the largest e4m3fn one.
GLOBAL_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)  # 2688


# ----------------------------------------------------------------------------- codecs
def e2m1_decode_scalar(code):
    """Value of one e2m1 nibble, from its bit fields."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = man * 0.5                      # subnormal: 2^(1-1) * (m / 2)
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man / 2.0)
    return sign * mag


def e4m3_decode_scalar(byte):
    """Value of one e4m3fn byte, from its bit fields (NaN for 0x7F / 0xFF)."""
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        mag = 2.0 ** -6 * (man / 8.0)        # subnormal
    else:
        mag = 2.0 ** (exp - 7) * (1.0 + man / 8.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_decode_scalar(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_decode_scalar(b) for b in range(256)], dtype=np.float64)


def e2m1_decode(codes):
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e4m3_decode(bytes_):
    return E4M3_TABLE[np.asarray(bytes_, dtype=np.uint8)]


def _nearest_code(mag, grid_vals, grid_codes):
    """Round non-negative magnitudes to the nearest grid value.

    ``grid_vals`` ascending, distinct, starting at 0; values above the last grid point
    saturate to it.  An exact tie between two neighbours goes to the code whose
    mantissa LSB is 0 ("even" code).  Returns the chosen codes.
    """
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid_vals, mag, side="left")          # first grid >= mag
    hi = np.clip(hi, 0, len(grid_vals) - 1)
    lo = np.clip(hi - 1, 0, len(grid_vals) - 1)
    d_lo = np.abs(mag - grid_vals[lo])
    d_hi = np.abs(grid_vals[hi] - mag)
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    pick_hi = np.where(tie, (grid_codes[hi] & 1) == 0, pick_hi)
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid_vals[-1], len(grid_vals) - 1, idx)  # saturate
    return grid_codes[idx]


_E2M1_POS_CODES = np.arange(8, dtype=np.int64)
_E2M1_POS_VALS = E2M1_TABLE[:8]
_E4M3_POS_CODES = np.array([b for b in range(0x7F)], dtype=np.int64)   # 0x00..0x7E finite
_E4M3_POS_VALS = E4M3_TABLE[:0x7F]


def e2m1_encode(vals):
    """Nearest e2m1 code, ties to even, saturating at 6, sign kept (-0 -> 0x8)."""
    vals = np.asarray(vals, dtype=np.float64)
    codes = _nearest_code(np.abs(vals), _E2M1_POS_VALS, _E2M1_POS_CODES)
    return (codes | np.where(np.signbit(vals), 0x8, 0)).astype(np.uint8)


def e4m3_encode(vals):
    """Nearest e4m3fn code, ties to even, saturating at 448, sign kept."""
    vals = np.asarray(vals, dtype=np.float64)
    codes = _nearest_code(np.abs(vals), _E4M3_POS_VALS, _E4M3_POS_CODES)
    return (codes | np.where(np.signbit(vals), 0x80, 0)).astype(np.uint8)


# ----------------------------------------------------------------------------- bf16
def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact float32 values."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32)


def f64_to_bf16_bits(vals):
    """Round float64 values straight to bf16 (8 significant bits), nearest-even.

    Done with frexp/rint on the float64 value itself (no detour through float32, which
    would round twice).  bf16 has float32's exponent range: normals down to 2^-126,
    subnormals in steps of 2^-133, overflow to infinity.
    """
    v = np.asarray(vals, dtype=np.float64)
    finite = np.isfinite(v)
    mant, exp = np.frexp(np.where(finite, v, 0.0))        # v = mant * 2^exp, |mant| in [0.5,1)
    # quantum of the 8-significant-bit grid at this binade, floored at the subnormal step
    q_exp = np.maximum(exp - 8, -133)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(v / q) * q                                 # np.rint: ties to even
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    out = np.where(finite, r, v)
    f32 = np.asarray(out.astype(np.float32))                            # exact: r is on the bf16 grid
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    return bits


# ----------------------------------------------------------------------------- quantizer
def quantize_row(x):
    """Quantize one activation row to NVFP4 with a per-row fp32 global.

    Follows the two-level NVFP4 reading (the pages name the format but print no
    quantizer; the readings are listed in the design notes):
      amax = max|x|;  gs = amax / 2688 (or 1 if amax == 0)
      per 16-block:   bmax = max|x_b|;  sf = bmax / (6 * gs);  sb = e4m3(sf)
                      d = e4m3_value(sb) * gs
      per element:    code = e2m1(x / d), or 0x0 for the whole block when d == 0
    All arithmetic in float32, in exactly this order; the nibble of the even element
    goes in the low half of each byte.  The row global is NOT folded into the codes:
    value(k) = e2m1_value(code_k) * e4m3_value(sb_block(k)) * gs.

    Returns (nibble_bytes uint8 [K/2], scale_bytes uint8 [K/16], gs float32).
    """
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[0]
    assert K % 16 == 0
    amax = np.float32(np.max(np.abs(x))) if K else np.float32(0)
    gs = np.float32(amax / GLOBAL_DIVISOR) if amax > 0 else np.float32(1.0)
    xb = x.reshape(-1, 16)                                   # one row per 16-block
    bmax = np.max(np.abs(xb), axis=1).astype(np.float32)
    t = np.float32(np.float32(6.0) * gs)
    sf = (bmax / t).astype(np.float32)                       # float32 division
    scales = e4m3_encode(sf.astype(np.float64))
    sd = e4m3_decode(scales).astype(np.float32)              # exact
    d = (sd * gs).astype(np.float32)                         # float32 product
    zero_block = d == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xb / np.where(zero_block, np.float32(1.0), d)[:, None]).astype(np.float32)
    codes = e2m1_encode(q.astype(np.float64))
    codes[zero_block, :] = 0
    codes = codes.reshape(-1)
    nib = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return nib, scales.astype(np.uint8), gs


def quantize_rows(x_rows):
    """``quantize_row`` applied to each row of a [R, K] float32 array."""
    x_rows = np.asarray(x_rows, dtype=np.float32)
    R, K = x_rows.shape
    q = np.zeros((R, K // 2), dtype=np.uint8)
    s = np.zeros((R, K // 16), dtype=np.uint8)
    g = np.zeros(R, dtype=np.float32)
    for i in range(R):
        q[i], s[i], g[i] = quantize_row(x_rows[i])
    return q, s, g


def unpack_nibbles(nib):
    """[..., K/2] bytes -> [..., K] e2m1 codes; the even element sits in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    out = np.empty(nib.shape[:-1] + (nib.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = nib & 0xF
    out[..., 1::2] = nib >> 4
    return out


def dequantize(nib, scales):
    """Exact float64 values e2m1(code) * e4m3(scale) of an NVFP4 matrix [..., K].

    The global (row or projection) is not applied.  Every such product is exactly
    representable in float64 (and in bf16 / f16), so this step has no rounding.
    """
    codes = unpack_nibbles(nib)
    vals = e2m1_decode(codes)
    sc = e4m3_decode(scales)
    return vals * np.repeat(sc, 16, axis=-1)
